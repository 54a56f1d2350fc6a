"""Host-side checks of the C ABI (no GPU needed, nothing is launched).

* libbased.so loads and exports every function include/based.h declares;
* argument validation returns the documented status before any launch
  (every call here is built to fail validation, so no device memory is
  touched);
* the product package never imports the oracle and fails loudly when the
  library is missing.
"""
import ast
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "based.h")
PKG = os.path.join(ROOT, "linear_attention_sequence_taylor_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    from linear_attention_sequence_taylor_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from linear_attention_sequence_taylor_amd import build

        build.build(verbose=False)
    return _lib.lib()


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for want in ("based_prefill", "based_decode_step", "swa_forward", "swa_cache_fill", "swa_decode_step",
                 "based_hybrid_prefill", "based_hybrid_prefill_workspace_bytes", "based_prefill_backward", "based_prefill_backward_workspace_bytes",
                 "based_swa_backward", "based_swa_backward_workspace_bytes",
                 "based_num_features", "based_prefill_workspace_bytes", "based_status_string"):
        assert want in names, names


def test_every_declared_symbol_is_exported(lib):
    from linear_attention_sequence_taylor_amd import _lib

    names = _declared_functions()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in based.h but not exported"
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with the header"


def test_header_is_plain_c_and_links(lib, tmp_path):
    """include/based.h compiles as C99 and as C++, and a C program linked
    against libbased.so (no Python) calls its host-only functions."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "use.c"
    src.write_text(
        '#include <stdio.h>\n#include "based.h"\n'
        "int main(void) {\n"
        '  printf("%d %d %s\\n", based_num_features(16), based_num_features(32), based_status_string(BASED_E_INVALID));\n'
        '  printf("%zu\\n", based_prefill_backward_workspace_bytes(1, 1, 64, 16, 64));\n'
        "  return 0;\n}\n")
    inc = os.path.join(ROOT, "include")
    for comp, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        subprocess.run([comp, std, "-Wall", "-Werror", "-fsyntax-only", "-x", "c" if comp == "gcc" else "c++",
                        "-I", inc, str(src)], check=True)
    exe = tmp_path / "use"
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe), "-L", PKG, "-lbased",
                    "-Wl,-rpath," + PKG], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.split("\n")
    assert out[0].split()[:2] == ["273", "1057"] and "INVALID" in out[0]
    assert int(out[1]) == lib.based_prefill_backward_workspace_bytes(1, 1, 64, 16, 64) > 0


def test_num_features_and_strings(lib):
    assert lib.based_num_features(16) == 273
    assert lib.based_num_features(8) == 73
    assert lib.based_num_features(0) == -1
    for s in range(5):
        assert lib.based_status_string(s)
    assert b"TOO_LARGE" in lib.based_status_string(4)
    assert b"UNKNOWN" in lib.based_status_string(99)


def test_workspace_bytes_host_only(lib):
    assert lib.based_prefill_workspace_bytes(1, 1, 256, 16, 64) >= 0
    assert lib.based_prefill_workspace_bytes(0, 1, 256, 16, 64) == 0
    assert lib.based_prefill_workspace_bytes(1, 1, 256, 8, 64) == 0
    assert lib.based_prefill_workspace_bytes(1, 1, 2**31 - 1, 16, 64) == 0
    # the fp32 matrix-core path: 32 heads x 4 groups of 16 columns fill half
    # the chip, so each head runs as 2 segments, one slot of F (d_v + 1)
    # floats (rounded up to 64) per (head, segment)
    F = 1 + 32 + 32 * 32
    slot = (F * 65 + 63) // 64 * 64
    assert lib.based_prefill_workspace_bytes(2, 16, 2048, 32, 64) == 32 * 2 * slot * 4
    assert lib.based_prefill_workspace_bytes(8, 16, 2048, 32, 64) == 0  # 512 groups: no split
    assert lib.based_prefill_workspace_bytes(2, 16, 500, 32, 64) == 0   # under 16 chunks: no split
    # d_feat 16 covers the bf16 plan and the fp32 path, whichever runs
    assert lib.based_prefill_workspace_bytes(1, 2, 4096, 16, 64) >= lib.based_prefill_workspace_bytes(1, 2, 4096, 8, 64)
    assert lib.based_hybrid_prefill_workspace_bytes(2, 16, 2048, 32, 64) == 32 * 2 * slot * 4


# Fake, never-dereferenced device addresses; each call below fails validation.
# Should a regression let one through, it would launch on these addresses:
# the calls run only where no HIP device is visible (counting devices does
# not initialise one).
def _hip_device_visible():
    try:
        import torch

        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


fake_addresses = pytest.mark.skipif(_hip_device_visible(), reason="fake device addresses: host-only check")

A = 0x7F0000000000
B_ = 0x7F1000000000
C = 0x7F2000000000
Y = 0x7F3000000000
S = 0x7F4000000000
Z = 0x7F5000000000


def _prefill(lib, **kw):
    a = dict(q=A, k=B_, v=C, dtype=1, B=1, H=1, L=64, d=16, dv=64, chunk=64, eps=1e-6, y=Y, S=S, z=Z,
             init=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.based_prefill(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"], a["d"], a["dv"],
                             a["chunk"], a["eps"], a["y"], a["S"], a["z"], a["init"], a["ws"], a["wsb"],
                             a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(y=None), 1), (dict(S=None), 1), (dict(z=None), 1),
    (dict(q=A + 2), 1), (dict(y=Y + 4), 1),
    (dict(dtype=7), 1), (dict(B=0), 1), (dict(H=-1), 1), (dict(L=0), 1),
    (dict(B=1 << 20, H=1 << 20), 1), (dict(chunk=0), 1), (dict(eps=float("nan")), 1),
    (dict(L=2**31 - 1), 1), (dict(L=2**31 - 1023), 1), (dict(B=1 << 10, H=1 << 10, L=1 << 21), 1),
    (dict(B=1 << 14, H=(1 << 13) + 1, L=1), 1),
    (dict(d=12), 2), (dict(d=64), 2), (dict(dv=96), 2), (dict(chunk=32), 2), (dict(dtype=0, chunk=48), 2),
    (dict(d=8, chunk=48), 2),
    (dict(y=A), 1), (dict(S=Y), 1), (dict(z=S + 64), 1),
    # a workspace overlapping y (bf16 plan) or S (fp32 path, d' 32), within
    # the part the call's plan may use
    (dict(H=2, L=4096, ws=Y + 256, wsb=1 << 30), 1),
    (dict(dtype=0, d=32, H=2, L=4096, ws=S - (1 << 20), wsb=1 << 30), 1),
])
@fake_addresses
def test_prefill_rejects(lib, kw, want):
    assert _prefill(lib, **kw) == want


def _decode(lib, **kw):
    a = dict(q=A, k=B_, v=C, dtype=1, B=2, H=3, d=16, dv=128, eps=1e-6, S=S, z=Z, y=Y, stream=None)
    a.update(kw)
    return lib.based_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["d"], a["dv"],
                                 a["eps"], a["S"], a["z"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(v=None), 1), (dict(S=S + 8), 1), (dict(B=0), 1), (dict(eps=float("inf")), 1),
    (dict(d=20), 2), (dict(dv=32), 2), (dict(y=S), 1), (dict(z=S + 16), 1), (dict(dtype=-1), 1),
])
@fake_addresses
def test_decode_rejects(lib, kw, want):
    assert _decode(lib, **kw) == want


def _swa(lib, **kw):
    a = dict(q=A, k=B_, v=C, dtype=1, B=1, H=2, L=100, dqk=64, dv=64, window=64, scale=0.125, add=None,
             y=Y, stream=None)
    a.update(kw)
    return lib.swa_forward(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"], a["dqk"],
                           a["dv"], a["window"], a["scale"], a["add"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(k=None), 1), (dict(add=S + 4), 1), (dict(window=0), 1), (dict(scale=float("nan")), 1),
    (dict(L=0), 1), (dict(dqk=32), 2), (dict(dv=96), 2), (dict(dv=32), 2), (dict(dqk=128), 2),
    (dict(y=A), 1), (dict(add=Y + 256), 1), (dict(L=2**31 - 1), 1), (dict(L=2**31 - 64), 1),
    (dict(dv=128, y=C + 64), 1),
])
@fake_addresses
def test_swa_rejects(lib, kw, want):
    assert _swa(lib, **kw) == want


def _swa_dec(lib, **kw):
    a = dict(q=A, k=B_, v=C, dtype=1, B=2, H=3, dqk=64, dv=64, window=64, scale=0.125, pos=S, kc=Y, vc=Z,
             add=None, y=S + (1 << 20), stream=None)
    a.update(kw)
    return lib.swa_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["B"], a["H"], a["dqk"], a["dv"],
                               a["window"], a["scale"], a["pos"], a["kc"], a["vc"], a["add"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(pos=None), 1), (dict(kc=None), 1), (dict(y=None), 1), (dict(pos=S + 4), 1),
    (dict(kc=Y + 8), 1), (dict(dtype=3), 1), (dict(B=0), 1), (dict(window=0), 1), (dict(scale=float("inf")), 1),
    (dict(dqk=32), 2), (dict(dv=96), 2), (dict(vc=Y + 64), 1), (dict(y=Y), 1),
    (dict(kc=A), 1), (dict(y=S), 1), (dict(add=S + (1 << 20) + 16), 1),
    # a wide window's key ring (3 MiB) reaching into the value ring
    (dict(window=4096, vc=Y + (1 << 20)), 1),
])
@fake_addresses
def test_swa_decode_rejects(lib, kw, want):
    assert _swa_dec(lib, **kw) == want


def _swa_fill(lib, **kw):
    a = dict(k=A, v=B_, dtype=1, B=1, H=2, L=100, dqk=64, dv=64, window=64, kc=Y, vc=Z, stream=None)
    a.update(kw)
    return lib.swa_cache_fill(a["k"], a["v"], a["dtype"], a["B"], a["H"], a["L"], a["dqk"], a["dv"], a["window"],
                              a["kc"], a["vc"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(k=None), 1), (dict(vc=None), 1), (dict(kc=Y + 2), 1), (dict(L=0), 1), (dict(window=0), 1),
    (dict(dqk=8), 2), (dict(dv=32), 2), (dict(vc=Y + 64), 1), (dict(kc=A), 1),
    (dict(L=2**31 - 1), 1),
])
@fake_addresses
def test_swa_fill_rejects(lib, kw, want):
    assert _swa_fill(lib, **kw) == want


V_ = 0x7F6000000000


def _hyb(lib, **kw):
    a = dict(q=A, k=B_, qw=C, kw=C + (1 << 32), v=V_, dtype=1, B=1, H=2, L=100, d=16, dqk=64, dv=64, chunk=64,
             eps=1e-6, window=64, scale=0.125, path=0, y=Y, S=S, z=Z, init=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.based_hybrid_prefill(a["q"], a["k"], a["qw"], a["kw"], a["v"], a["dtype"], a["B"], a["H"], a["L"],
                                    a["d"], a["dqk"], a["dv"], a["chunk"], a["eps"], a["window"], a["scale"],
                                    a["path"], a["y"], a["S"], a["z"], a["init"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(qw=None), 1), (dict(kw=None), 1), (dict(v=None), 1), (dict(z=None), 1),
    (dict(y=Y + 4), 1), (dict(kw=C + 8), 1), (dict(ws=Z + (1 << 30) + 4), 1), (dict(dtype=5), 1), (dict(L=0), 1),
    (dict(eps=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(window=0), 1), (dict(d=12), 2),
    (dict(dv=96), 2), (dict(dqk=8), 2), (dict(path=1, window=200), 2), (dict(chunk=32), 2), (dict(y=A), 1),
    (dict(S=Y), 1), (dict(z=V_), 1), (dict(y=C + (1 << 32)), 1), (dict(path=3), 1), (dict(path=-1), 1),
    (dict(path=1, dqk=16), 2), (dict(path=1, dtype=0), 2), (dict(path=1, window=65), 2), (dict(path=1, d=8), 2),
    # a workspace overlapping the window keys, within the part a plan may use
    (dict(L=4096, ws=C + (1 << 32) + 256, wsb=1 << 30), 1),
])
@fake_addresses
def test_hybrid_rejects(lib, kw, want):
    assert _hyb(lib, **kw) == want


def test_hybrid_workspace_bytes(lib):
    # at least what the linear branch alone asks for; zero where no matrix-core plan exists
    for L in (100, 8192, 65536):
        assert lib.based_hybrid_prefill_workspace_bytes(4, 16, L, 16, 64) >= lib.based_prefill_workspace_bytes(
            4, 16, L, 16, 64)
        assert lib.based_hybrid_prefill_workspace_bytes(4, 16, L, 16, 128) >= lib.based_prefill_workspace_bytes(
            4, 16, L, 16, 128)
    assert lib.based_hybrid_prefill_workspace_bytes(4, 16, 8192, 16, 96) == 0
    assert lib.based_hybrid_prefill_workspace_bytes(4, 16, 8192, 8, 64) == 0


def _bwd(lib, **kw):
    a = dict(q=A, k=B_, v=C, dy=Y, dtype=1, B=1, H=2, L=100, d=16, dv=64, eps=1e-6, form=0, dq=S, dk=S + (1 << 20),
             dvo=S + (2 << 20), ws=Z, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.based_prefill_backward(a["q"], a["k"], a["v"], a["dy"], a["dtype"], a["B"], a["H"], a["L"], a["d"],
                                      a["dv"], a["eps"], a["form"], a["dq"], a["dk"], a["dvo"], a["ws"], a["wsb"],
                                      a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(dy=None), 1), (dict(ws=None), 1), (dict(dq=S + 4), 1), (dict(wsb=100), 1),
    (dict(dtype=5), 1), (dict(L=0), 1), (dict(eps=float("nan")), 1), (dict(d=12), 2), (dict(dv=32), 2),
    (dict(dq=A), 1), (dict(dk=S), 1), (dict(ws=S + (2 << 20)), 1), (dict(dvo=Y), 1),
    # the form: unknown values, and the chunked form outside bf16 / d' 16
    (dict(form=3), 1), (dict(form=-1), 1), (dict(form=2, dtype=0), 2), (dict(form=2, d=8), 2),
    (dict(form=2, d=8, dv=128), 2),
    # the chunked form's workspace is larger than the direct form's at d_v 64
    # and the same at d_v 128
    (dict(form=2, wsb=2 * 100 * 65 * 4), 1), (dict(form=2, dv=128, wsb=2 * 100 * 65 * 4), 1),
])
@fake_addresses
def test_backward_rejects(lib, kw, want):
    assert _bwd(lib, **kw) == want


def _swabwd(lib, **kw):
    a = dict(q=A, k=B_, v=C, dy=Y, dtype=1, B=1, H=2, L=100, dqk=64, dv=64, window=64, scale=0.125, dq=S,
             dk=S + (1 << 20), dvo=S + (2 << 20), ws=Z, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.based_swa_backward(a["q"], a["k"], a["v"], a["dy"], a["dtype"], a["B"], a["H"], a["L"], a["dqk"],
                                  a["dv"], a["window"], a["scale"], a["dq"], a["dk"], a["dvo"], a["ws"], a["wsb"],
                                  a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(dy=None), 1), (dict(ws=None), 1), (dict(dq=S + 4), 1), (dict(wsb=100), 1),
    (dict(dtype=5), 1), (dict(L=0), 1), (dict(scale=float("nan")), 1), (dict(window=0), 1),
    (dict(dq=A), 1), (dict(dk=S), 1), (dict(ws=S + (2 << 20)), 1), (dict(dvo=Y), 1),
    # well formed, outside what the kernels implement
    (dict(dtype=0), 2), (dict(dqk=16), 2), (dict(dv=96), 2), (dict(window=65), 2),
])
@fake_addresses
def test_swa_backward_rejects(lib, kw, want):
    assert _swabwd(lib, **kw) == want


def test_swa_backward_workspace_bytes(lib):
    assert lib.based_swa_backward_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 16
    assert lib.based_swa_backward_workspace_bytes(2, 3, 0) == 0


def test_backward_workspace_bytes(lib):
    # direct form: g and h; d' 16 also covers the chunked form's per-segment
    # states (the same for both d_v: one 64-column pass at a time)
    assert lib.based_prefill_backward_workspace_bytes(2, 3, 100, 16, 128) >= 2 * 3 * 100 * 129 * 4
    for L in (100, 4096, 65536):
        assert lib.based_prefill_backward_workspace_bytes(2, 3, L, 16, 128) >= \
            lib.based_prefill_backward_workspace_bytes(2, 3, L, 16, 64)
    assert lib.based_prefill_backward_workspace_bytes(2, 3, 100, 8, 128) == 2 * 3 * 100 * 129 * 4
    assert lib.based_prefill_backward_workspace_bytes(2, 3, 100, 8, 64) == 2 * 3 * 100 * 65 * 4
    assert lib.based_prefill_backward_workspace_bytes(2, 3, 100, 16, 64) > 2 * 3 * 100 * 65 * 4
    assert lib.based_prefill_backward_workspace_bytes(2, 3, 100, 12, 64) == 0
    assert lib.based_prefill_backward_workspace_bytes(0, 3, 100, 16, 64) == 0


def test_product_never_imports_oracle():
    for dirpath, _, files in os.walk(PKG):
        for fn in files:
            if not fn.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, fn)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert not any(a.name.split(".")[0] == "oracle" for a in node.names), fn
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", fn
    for dirpath, _, files in os.walk(os.path.join(PKG, "csrc")):
        for fn in files:
            assert "oracle" not in open(os.path.join(dirpath, fn)).read().lower(), fn


def test_missing_library_fails_loudly(monkeypatch):
    from linear_attention_sequence_taylor_amd import _lib

    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libbased.so")
    with pytest.raises(ImportError):
        _lib.lib()


def test_build_flags_name_existing_sources():
    """Every per-source flag set in the build script names a source that is
    compiled (a misspelt name would silently drop its flags), and the
    packed-fp32 forms are off for all device code."""
    from linear_attention_sequence_taylor_amd import build

    sources = set(os.listdir(build.CSRC))
    assert set(build.SOURCE_FLAGS) <= sources
    assert all(name.endswith((".hip", ".cpp")) for name in build.SOURCE_FLAGS)
    assert "-packed-fp32-ops" in build.DEVICE_FLAGS
    # the scheduler choice per unit: the two hottest prefill instances under
    # the iterative ILP scheduler, the bf16 gradients under max-ilp, the
    # rest under the default one
    assert "-amdgpu-sched-strategy=iterative-ilp" in build.SOURCE_FLAGS["prefill_mfma_ilp.hip"]
    assert "-amdgpu-sched-strategy=max-ilp" in build.SOURCE_FLAGS["prefill_backward_mfma.hip"]
    assert "prefill_mfma.hip" not in build.SOURCE_FLAGS
