"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Bar (max-abs error as a multiple of the oracle output's RMS over the
compared tensor): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.  Full-size
workloads are run on the GPU exactly as the benchmark launches them; the
oracle then recomputes a sample of whole (batch, head) pairs, which is exact
because every (batch, head) is independent.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build()
    import linear_attention_sequence_taylor_amd as based  # noqa: F401  (fails loudly without the .so)

    assert torch.cuda.is_available(), "GPU tests need a HIP device"


def based_mod():
    import linear_attention_sequence_taylor_amd as based

    return based


def ratio(got, want):
    got = np.asarray(got.detach().cpu().double() if isinstance(got, torch.Tensor) else got, np.float64)
    want = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    return float(np.abs(got - want).max()) / rms


def report(name, r, tol):
    print(f"[parity] {name}: max_err/rms = {r:.3e} (bar {tol:.0e})", flush=True)
    assert r <= tol, f"{name}: {r:.3e} > {tol:.0e}"


def dev(*ts):
    return [t.to(DEV) for t in ts]


# ---------------------------------------------------------------- prefill
@pytest.mark.parametrize("L", [1, 17, 63, 64, 65, 130, 1000])
@pytest.mark.parametrize("dv", [64, 128])
def test_prefill_bf16_shapes(L, dv):
    based = based_mod()
    q, k, v = si.custom((2, 3, L, 16), (2, 3, L, dv), seed=500 + L + dv, scale=0.5)
    y, S, z = based.based_prefill(*dev(q, k, v))
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"prefill bf16 L={L} dv={dv} y", ratio(y, yo), 2e-2)
    report(f"prefill bf16 L={L} dv={dv} S", ratio(S, So), 2e-2)
    report(f"prefill bf16 L={L} dv={dv} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dv", [64, 128])
def test_prefill_f32_chunks(chunk, dv):
    based = based_mod()
    q, k, v = si.custom((1, 2, 100, 16), (1, 2, 100, dv), seed=600 + chunk, scale=1.0, dtype=torch.float32)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=chunk)
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"prefill f32 chunk={chunk} dv={dv} y", ratio(y, yo), 1e-4)
    report(f"prefill f32 chunk={chunk} dv={dv} S", ratio(S, So), 1e-4)
    report(f"prefill f32 chunk={chunk} dv={dv} z", ratio(z, zo), 1e-4)


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
def test_prefill_resume_from_state(dtype, tol):
    based = based_mod()
    L1, L2 = 130, 700  # the second call is long enough to be split into segments (bf16)
    q, k, v = si.custom((1, 4, L1 + L2, 16), (1, 4, L1 + L2, 64), seed=700, scale=0.5, dtype=dtype)
    qd, kd, vd = dev(q, k, v)
    _, S1, z1 = based.based_prefill(qd[:, :, :L1].contiguous(), kd[:, :, :L1].contiguous(),
                                    vd[:, :, :L1].contiguous())
    y2, S2, z2 = based.based_prefill(qd[:, :, L1:].contiguous(), kd[:, :, L1:].contiguous(),
                                     vd[:, :, L1:].contiguous(), initial_state=(S1, z1))
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"resume {dtype} y", ratio(y2, yo[:, :, L1:]), tol)
    report(f"resume {dtype} S", ratio(S2, So), tol)
    report(f"resume {dtype} z", ratio(z2, zo), tol)


@pytest.mark.parametrize("dtype,tol,d,L", [
    (torch.float32, 1e-4, 16, 1), (torch.float32, 1e-4, 32, 65), (torch.bfloat16, 2e-2, 8, 257),
    (torch.float32, 1e-4, 24, 130),
])
def test_prefill_fp32_path_initial_state(dtype, tol, d, L):
    """The fp32 matrix-core prefill (chunk 64, any feature dim) from an
    asymmetric carried state: outputs, and the state returned as the initial
    one plus this call's increment, row for row."""
    based = based_mod()
    F = 1 + d + d * d
    q, k, v = si.custom((1, 2, L, d), (1, 2, L, 64), seed=760 + d + L, scale=0.5, dtype=dtype)
    qp, kp, vp = si.custom((1, 2, 40, d), (1, 2, 40, 64), seed=762 + d, scale=0.5)
    _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
    S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
    g = torch.Generator().manual_seed(763 + d)
    P = torch.randn((1, 2, d, d, 64), generator=g)
    S0[:, :, 1 + d:] += 0.5 * (P - P.transpose(2, 3)).reshape(1, 2, d * d, 64)
    y, S, z = based.based_prefill(*dev(q, k, v), initial_state=tuple(dev(S0, z0)))
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    assert S.shape[2] == F
    report(f"fp32-path init-state {dtype} d={d} L={L} y", ratio(y, yo), tol)
    report(f"fp32-path init-state {dtype} d={d} L={L} S", ratio(S, So), tol)
    report(f"fp32-path init-state {dtype} d={d} L={L} z", ratio(z, zo), tol)


@pytest.mark.parametrize("L", [70, 900])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("ws", ["auto", "none"])
def test_prefill_random_initial_state(L, dv, ws):
    """An arbitrary (asymmetric) carried state: outputs see its symmetric
    part, the returned state is the initial one plus this call's increment.
    ws="none" hands over an empty workspace, which must fall back to a
    launch shape that needs none."""
    based = based_mod()
    q, k, v = si.custom((1, 3, L, 16), (1, 3, L, dv), seed=710 + L + dv, scale=0.5)
    # a reachable state (oracle state after a 50-token prefix, so every
    # denominator stays positive) plus an antisymmetric part in the pair rows
    qp, kp, vp = si.custom((1, 3, 50, 16), (1, 3, 50, dv), seed=712 + L, scale=0.5)
    _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
    S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
    g = torch.Generator().manual_seed(711 + L)
    P = torch.randn((1, 3, 16, 16, dv), generator=g)
    S0[:, :, 17:] += (P - P.transpose(2, 3)).reshape(1, 3, 256, dv)
    Pz = torch.randn((1, 3, 16, 16), generator=g)
    z0[:, :, 17:] += (Pz - Pz.transpose(2, 3)).reshape(1, 3, 256)
    kw = {} if ws == "auto" else {"workspace": torch.empty(0, dtype=torch.uint8, device=DEV)}
    y, S, z = based.based_prefill(*dev(q, k, v), initial_state=tuple(dev(S0, z0)), **kw)
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    report(f"init-state L={L} dv={dv} ws={ws} y", ratio(y, yo), 2e-2)
    report(f"init-state L={L} dv={dv} ws={ws} S", ratio(S, So), 2e-2)
    report(f"init-state L={L} dv={dv} ws={ws} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("dv", [64, 128])
def test_prefill_many_heads(dv):
    """Enough heads that each one runs unsplit in length (and, for d_v = 128,
    in wider column groups)."""
    based = based_mod()
    q, k, v = si.custom((2, 132, 70, 16), (2, 132, 70, dv), seed=720 + dv, scale=0.5)
    y, S, z = based.based_prefill(*dev(q, k, v))
    torch.cuda.synchronize()
    pick = [(0, 0), (0, 131), (1, 64), (1, 131)]
    for b, h in pick:
        sl = (slice(b, b + 1), slice(h, h + 1))
        yo, So, zo = oracle.la_recurrent(q[sl], k[sl], v[sl])
        report(f"many-heads dv={dv} ({b},{h}) y", ratio(y[sl], yo), 2e-2)
        report(f"many-heads dv={dv} ({b},{h}) S", ratio(S[sl], So), 2e-2)
        report(f"many-heads dv={dv} ({b},{h}) z", ratio(z[sl], zo), 2e-2)


@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("init", [False, True])
def test_prefill_long_few_heads(dv, init):
    """Few heads and a long ragged sequence: the launch takes 64-wide value
    groups and ~100 sequence segments of three chunks (state pass, prefix
    scan over segments, output pass), with and without a carried state."""
    based = based_mod()
    L = 64 * 300 + 17
    q, k, v = si.custom((1, 2, L, 16), (1, 2, L, dv), seed=730 + dv + init, scale=0.5)
    S0 = z0 = None
    kw = {}
    if init:
        qp, kp, vp = si.custom((1, 2, 50, 16), (1, 2, 50, dv), seed=731 + dv, scale=0.5)
        _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
        S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
        kw["initial_state"] = tuple(dev(S0, z0))
    y, S, z = based.based_prefill(*dev(q, k, v), **kw)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    report(f"long few-heads dv={dv} init={init} y", ratio(y, yo), 2e-2)
    report(f"long few-heads dv={dv} init={init} S", ratio(S, So), 2e-2)
    report(f"long few-heads dv={dv} init={init} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("L,H", [(300, 2), (2048, 4)])
def test_prefill_graph_replay(L, H):
    """Captured in a HIP graph (as the benchmark runs it), every replay gives
    the eager result bit for bit, with eager work and synchronisation in
    between replays.  (2048, 4) takes the segment split and its workspace."""
    based = based_mod()
    q, k, v = dev(*si.custom((1, H, L, 16), (1, H, L, 64), seed=810 + L, scale=0.5))
    nbytes = based.based_prefill_workspace_bytes(1, H, L, 64)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty(1, H, L, 64, device=DEV)
    S = torch.empty(1, H, 273, 64, device=DEV)
    z = torch.empty(1, H, 273, device=DEV)
    ref = [t.clone() for t in based.based_prefill(q, k, v, y=y, S=S, z=z, workspace=ws)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        based.based_prefill(q, k, v, y=y, S=S, z=z, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        based.based_prefill(q, k, v, y=y, S=S, z=z, workspace=ws)
    for rep in range(3):
        for t in (y, S, z):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip("ySz", (y, S, z), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager result"
        based.based_prefill(q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous())  # eager work
        torch.cuda.synchronize()


def test_prefill_deterministic():
    based = based_mod()
    q, k, v = dev(*si.custom((2, 2, 300, 16), (2, 2, 300, 64), seed=800, scale=0.5))
    a = [t.clone() for t in based.based_prefill(q, k, v)]
    b = based.based_prefill(q, k, v)
    for x, w in zip(a, b):
        assert torch.equal(x, w)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
@pytest.mark.parametrize("dv", [64, 128])
def test_decode_from_oracle_state(dtype, tol, dv):
    """One step from a state built by the oracle (independent of prefill)."""
    based = based_mod()
    L = 50
    q, k, v = si.custom((3, 2, L + 1, 16), (3, 2, L + 1, dv), seed=900 + dv, scale=1.0, dtype=dtype)
    _, S0, z0 = oracle.la_recurrent(q[:, :, :L], k[:, :, :L], v[:, :, :L], want_y=False)
    S_in = torch.from_numpy(S0).float()
    z_in = torch.from_numpy(z0).float()
    S, z = S_in.to(DEV), z_in.to(DEV)
    qt, kt, vt = (t[:, :, L].contiguous() for t in (q, k, v))
    y = based.based_decode_step(*dev(qt, kt, vt), S, z)
    yo, So, zo = oracle.decode_step(qt, kt, vt, S_in, z_in)
    report(f"decode {dtype} dv={dv} y", ratio(y, yo), tol)
    report(f"decode {dtype} dv={dv} S", ratio(S, So), tol)
    report(f"decode {dtype} dv={dv} z", ratio(z, zo), tol)


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
def test_prefill_then_decode_equals_longer_prefill(dtype, tol):
    based = based_mod()
    L1, T = 64 * 3 + 5, 40
    q, k, v = si.custom((2, 2, L1 + T, 16), (2, 2, L1 + T, 128), seed=1000, scale=1.0, dtype=dtype)
    qd, kd, vd = dev(q, k, v)
    _, S, z = based.based_prefill(qd[:, :, :L1].contiguous(), kd[:, :, :L1].contiguous(),
                                  vd[:, :, :L1].contiguous())
    ys = []
    for t in range(L1, L1 + T):
        ys.append(based.based_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                          vd[:, :, t].contiguous(), S, z).clone())
    got = torch.stack(ys, dim=2)
    yo = oracle.la_quadratic(q, k, v)
    report(f"prefill+decode {dtype}", ratio(got, yo[:, :, L1:]), tol)


# ---------------------------------------------------------------- window
@pytest.mark.parametrize("dqk", [16, 64])
@pytest.mark.parametrize("window", [1, 7, 64])
@pytest.mark.parametrize("L", [1, 50, 64, 129, 300])
def test_swa_bf16_shapes(dqk, window, L):
    based = based_mod()
    q, k, v = si.custom((1, 3, L, dqk), (1, 3, L, 64), seed=1100 + L + window, scale=1.0)
    scale = dqk ** -0.5
    y = based.swa_forward(*dev(q, k, v), window=window, scale=scale)
    report(f"swa bf16 dqk={dqk} w={window} L={L}", ratio(y, oracle.swa(q, k, v, window, scale)), 2e-2)


@pytest.mark.parametrize("dqk", [16, 64])
def test_swa_f32(dqk):
    based = based_mod()
    q, k, v = si.custom((2, 2, 200, dqk), (2, 2, 200, 64), seed=1200, scale=1.0, dtype=torch.float32)
    y = based.swa_forward(*dev(q, k, v), window=64, scale=dqk ** -0.5)
    report(f"swa f32 dqk={dqk}", ratio(y, oracle.swa(q, k, v, 64, dqk ** -0.5)), 1e-4)


def test_swa_add_modes():
    based = based_mod()
    q, k, v = si.custom((1, 2, 130, 64), (1, 2, 130, 64), seed=1300, scale=1.0)
    qd, kd, vd = dev(q, k, v)
    base = torch.randn(1, 2, 130, 64, generator=torch.Generator().manual_seed(5)).to(DEV)
    y_plain = based.swa_forward(qd, kd, vd)
    y_add = based.swa_forward(qd, kd, vd, add=base)
    y_inplace = base.clone()
    based.swa_forward(qd, kd, vd, add=y_inplace, y=y_inplace)
    assert torch.allclose(y_add, y_plain + base, rtol=0, atol=1e-6)
    assert torch.equal(y_inplace, y_add)


@pytest.mark.parametrize("dqk,add,window", [(64, False, 64), (16, True, 64), (64, True, 128), (16, False, 100)])
def test_swa_long_runs(dqk, add, window):
    """Many 64-query tiles per workgroup (B*H=128, 38 tiles a head: runs of
    10 tiles, the last one 8, ending in a ragged tile), so every slot
    rotation of the K/V/Q ring is used; two launches must agree bit for bit."""
    based = based_mod()
    B, H, L = 2, 64, 64 * 37 + 5
    q, k, v = si.custom((B, H, L, dqk), (B, H, L, 64), seed=1400 + dqk, scale=1.0)
    qd, kd, vd = dev(q, k, v)
    base = torch.randn(B, H, L, 64, generator=torch.Generator().manual_seed(6)) if add else None
    scale = dqk ** -0.5
    outs = [based.swa_forward(qd, kd, vd, window=window, scale=scale,
                              add=base.to(DEV) if add else None) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    heads = _sample_heads(B, H, 4, 3)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    want = oracle.swa(q[bi, hi], k[bi, hi], v[bi, hi], window, scale)
    if add:
        want = want + base[bi, hi].double().numpy()
    report(f"swa long runs dqk={dqk} add={add} w={window} (4 sampled heads)", ratio(outs[0][bi, hi], want), 2e-2)


@pytest.mark.parametrize("L", [2**23 - 37, 2**23 + 29])
def test_swa_longest_heads(L):
    """Heads at the 32-bit offset limit of the matrix-core window kernel
    (L * 256 bytes of fp32 output per head): just below it that kernel runs,
    just above it the fp32-accumulating vector kernel takes bf16 inputs.  A
    4096-row random block is repeated along L; sampled queries are checked
    against the oracle on their own 64-key slice (a query sees nothing else)."""
    based = based_mod()
    P = 4096
    blocks = si.custom((1, 1, P, 16), (1, 1, P, 64), seed=1500, scale=1.0)
    reps = (L + P - 1) // P
    q, k, v = (t.repeat(1, 1, reps, 1)[:, :, :L].contiguous() for t in blocks)
    y = based.swa_forward(*dev(q, k, v), window=64, scale=0.25)
    torch.cuda.synchronize()
    rows = [0, 5, 63, 64, 4095, 4096, L // 2 + 7, 2**23 - 100, L - 65, L - 2, L - 1]
    got = torch.stack([y[0, 0, i] for i in rows]).cpu()
    want = np.stack([oracle.swa(q[:, :, max(0, i - 63):i + 1], k[:, :, max(0, i - 63):i + 1],
                                v[:, :, max(0, i - 63):i + 1], 64, 0.25)[0, 0, -1] for i in rows])
    report(f"swa longest head L={L} ({len(rows)} sampled queries)", ratio(got, want), 2e-2)


# ---------------------------------------------------------------- other feature and window sizes
@pytest.mark.parametrize("d", [8, 24, 32])
@pytest.mark.parametrize("dtype,tol,chunk,dv", [(torch.bfloat16, 2e-2, 64, 64), (torch.float32, 1e-4, 64, 128),
                                                (torch.float32, 1e-4, 16, 64)])
def test_prefill_feature_dims(d, dtype, tol, chunk, dv):
    """Feature dims 8, 24 and 32 (F = 73, 601, 1057 rows), ragged length."""
    based = based_mod()
    q, k, v = si.custom((1, 2, 130, d), (1, 2, 130, dv), seed=1800 + d + dv + chunk, scale=0.5, dtype=dtype)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=chunk)
    torch.cuda.synchronize()
    assert S.shape[-2] == 1 + d + d * d
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"prefill d={d} {dtype} chunk={chunk} dv={dv} y", ratio(y, yo), tol)
    report(f"prefill d={d} {dtype} chunk={chunk} dv={dv} S", ratio(S, So), tol)
    report(f"prefill d={d} {dtype} chunk={chunk} dv={dv} z", ratio(z, zo), tol)


@pytest.mark.parametrize("d", [8, 24, 32])
@pytest.mark.parametrize("dtype,tol,dv", [(torch.bfloat16, 2e-2, 128), (torch.float32, 1e-4, 64)])
def test_prefill_then_decode_feature_dims(d, dtype, tol, dv):
    """Prefill then next-token steps with feature dims 8, 24, 32: the steps
    equal the longer sequence's outputs (the state handoff at 1 + d + d^2 rows)."""
    based = based_mod()
    L1, T = 70, 6
    q, k, v = si.custom((2, 2, L1 + T, d), (2, 2, L1 + T, dv), seed=1850 + d + dv, scale=1.0, dtype=dtype)
    qd, kd, vd = dev(q, k, v)
    _, S, z = based.based_prefill(qd[:, :, :L1].contiguous(), kd[:, :, :L1].contiguous(), vd[:, :, :L1].contiguous())
    ys = [based.based_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                  S, z).clone() for t in range(L1, L1 + T)]
    yo = oracle.la_quadratic(q, k, v)
    report(f"prefill+decode d={d} {dtype} dv={dv}", ratio(torch.stack(ys, dim=2), yo[:, :, L1:]), tol)


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
@pytest.mark.parametrize("dqk", [16, 64])
@pytest.mark.parametrize("window,L", [(65, 129), (100, 300), (128, 1), (128, 300)])
def test_swa_wide_windows(dtype, tol, dqk, window, L):
    """Windows over 64 keys (up to 128, the pages' other design point)."""
    based = based_mod()
    q, k, v = si.custom((1, 3, L, dqk), (1, 3, L, 64), seed=1900 + window + L + dqk, scale=1.0, dtype=dtype)
    scale = dqk ** -0.5
    y = based.swa_forward(*dev(q, k, v), window=window, scale=scale)
    report(f"swa {dtype} dqk={dqk} w={window} L={L}", ratio(y, oracle.swa(q, k, v, window, scale)), tol)


# ---------------------------------------------------------------- backward
@pytest.mark.parametrize("dtype,tol,B,H,L,d,dv", [
    (torch.bfloat16, 2e-2, 1, 2, 130, 16, 64), (torch.float32, 1e-4, 1, 2, 130, 16, 64),
    (torch.float32, 1e-4, 1, 2, 70, 32, 128), (torch.bfloat16, 2e-2, 2, 1, 257, 8, 64),
    (torch.bfloat16, 2e-2, 1, 3, 33, 24, 128), (torch.bfloat16, 2e-2, 2, 2, 200, 16, 128),
    (torch.bfloat16, 2e-2, 1, 1, 64, 16, 64), (torch.bfloat16, 2e-2, 1, 2, 3, 16, 64),
    (torch.float32, 1e-4, 1, 2, 257, 8, 64), (torch.float32, 1e-4, 2, 1, 200, 24, 128),
    (torch.float32, 1e-4, 1, 1, 600, 16, 128), (torch.float32, 1e-4, 1, 2, 65, 32, 64),
    (torch.bfloat16, 2e-2, 1, 2, 190, 32, 128), (torch.float32, 1e-4, 1, 1, 5, 24, 64),
])
def test_backward_matches_oracle(dtype, tol, B, H, L, d, dv):
    """dq, dk, dv of the prefill output for a seeded upstream gradient, against
    the oracle's chain rule (itself pinned to autograd and finite differences)."""
    based = based_mod()
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=2200 + L + d + dv, scale=0.5, dtype=dtype)
    dy = torch.randn(B, H, L, dv, generator=torch.Generator().manual_seed(2201 + L))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV))
    torch.cuda.synchronize()
    oq, ok, ov = oracle.la_backward(q, k, v, dy)
    report(f"backward {dtype} L={L} d={d} dv={dv} dq", ratio(dq, oq), tol)
    report(f"backward {dtype} L={L} d={d} dv={dv} dk", ratio(dk, ok), tol)
    report(f"backward {dtype} L={L} d={d} dv={dv} dv", ratio(dv_, ov), tol)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_single_token(dtype):
    """L = 1: y_0 = v_0 a/(a + eps), so dv_0 = dy_0 a/(a + eps) and dq, dk are
    of order eps: they come out of the cancellation of terms of order
    |dy||v|, and fp32 gives them to rounding noise of those terms."""
    based = based_mod()
    q, k, v = si.custom((2, 2, 1, 16), (2, 2, 1, 128), seed=2250, scale=1.0, dtype=dtype)
    dy = torch.randn(2, 2, 1, 128, generator=torch.Generator().manual_seed(2251))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV))
    oq, ok, ov = oracle.la_backward(q, k, v, dy)
    report(f"backward L=1 {dtype} dv", ratio(dv_, ov), 1e-4)
    noise = 1e-5 * float(dy.norm(dim=-1).max() * v.float().norm(dim=-1).max() * k.float().norm(dim=-1).max())
    assert float(dq.abs().max()) <= noise and float(dk.abs().max()) <= noise, (dq.abs().max(), dk.abs().max(), noise)
    assert np.abs(oq).max() <= noise and np.abs(ok).max() <= noise


def test_workload_prefill_360m_backward():
    """Gradients over the 360M-shaped layer (B=8, H=16, L=2048), 2 sampled heads."""
    based = based_mod()
    wl = si.WORKLOADS["prefill_360m"]
    q, k, v = si.linear_inputs(wl)
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2300))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), eps=wl.eps)
    torch.cuda.synchronize()
    heads = _sample_heads(wl.B, wl.H, 2, 5)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    oq, ok, ov = oracle.la_backward(q[bi, hi], k[bi, hi], v[bi, hi], dy[bi, hi], eps=wl.eps)
    report("prefill_360m backward dq (2 sampled heads)", ratio(dq[bi, hi], oq), wl.tol)
    report("prefill_360m backward dk (2 sampled heads)", ratio(dk[bi, hi], ok), wl.tol)
    report("prefill_360m backward dv (2 sampled heads)", ratio(dv_[bi, hi], ov), wl.tol)


# ---------------------------------------------------------------- window decode
def _nan_cache(B, H, window, d, dtype):
    return torch.full((B, H, window, d), float("nan"), dtype=dtype, device=DEV)


@pytest.mark.parametrize("dtype,dqk,dv,window,L", [
    (torch.bfloat16, 64, 64, 64, 100), (torch.bfloat16, 16, 128, 64, 10), (torch.bfloat16, 64, 128, 7, 30),
    (torch.bfloat16, 64, 64, 64, 0), (torch.float32, 64, 64, 64, 64), (torch.float32, 16, 128, 1, 5),
    (torch.float32, 64, 128, 33, 200), (torch.bfloat16, 64, 128, 128, 200), (torch.float32, 16, 64, 100, 10),
    (torch.bfloat16, 64, 64, 128, 0),
])
def test_swa_decode_continues_window(dtype, dqk, dv, window, L):
    """Ring filled from a prefix (two sequences, prefixes L and L + 5; none
    for L = 0, which starts decoding at position 0 on an empty ring), then
    2*window + 3 next-token steps.  Every step's output is compared with the
    oracle's brute-force window attention over the whole sequence at that
    position; the caches start as NaN, so reading a slot that does not hold
    one of the last `window` tokens would show.  The final caches must hold
    exactly the oracle's ring."""
    based = based_mod()
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    B, H, lag = 2, 3, 5
    T = 2 * window + 3
    n = L + lag + T
    q, k, v = si.custom((B, H, n, dqk), (B, H, n, dv), seed=1600 + dqk + dv + window + L, scale=1.0, dtype=dtype)
    qd, kd, vd = dev(q, k, v)
    scale = dqk ** -0.5
    full = oracle.swa(q, k, v, window, scale)
    kc, vc = _nan_cache(B, H, window, dqk, dtype), _nan_cache(B, H, window, dv, dtype)
    okc = np.full((B, H, window, dqk), np.nan)
    ovc = np.full((B, H, window, dv), np.nan)
    starts = [L, L + lag]
    for b, L0 in enumerate(starts):
        if L0 > 0:
            based.swa_cache_fill(kd[b:b + 1, :, :L0].contiguous(), vd[b:b + 1, :, :L0].contiguous(),
                                 window=window, k_cache=kc[b:b + 1], v_cache=vc[b:b + 1])
            okc[b], ovc[b] = oracle.swa_cache_fill(k[b:b + 1, :, :L0], v[b:b + 1, :, :L0], window,
                                                   okc[b:b + 1], ovc[b:b + 1])
    got, want = [], []
    for t in range(T):
        p = [L0 + t for L0 in starts]
        pick = lambda x: torch.stack([x[b, :, p[b]] for b in range(B)]).contiguous()
        pos = torch.tensor(p, dtype=torch.int64, device=DEV)
        got.append(based.swa_decode_step(pick(qd), pick(kd), pick(vd), kc, vc, pos, scale=scale).cpu())
        want.append(np.stack([full[b, :, p[b]] for b in range(B)]))
        _, okc, ovc = oracle.swa_decode_step(pick(q), pick(k), pick(v), okc, ovc, p, window, scale)
    report(f"swa decode {dtype} dqk={dqk} dv={dv} w={window} L={L} ({T} steps)",
           ratio(torch.stack(got), np.stack(want)), tol)
    np.testing.assert_array_equal(kc.double().cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.double().cpu().numpy(), ovc)


def test_swa_decode_add_and_invalid_position():
    """add (fused sum, in place on y); a negative position gives NaN outputs
    for its sequence and leaves that sequence's cache untouched."""
    based = based_mod()
    B, H, window = 2, 2, 64
    q, k, v = si.custom((B, H, 64), (B, H, 64), seed=1700)
    kp, vp = si.custom((B, H, 80, 64), (B, H, 80, 64), seed=1701)[1:]
    kc, vc = based.swa_cache_fill(*dev(kp, vp), window=window)
    kc0, vc0 = kc.clone(), vc.clone()
    base = torch.randn(B, H, 64, generator=torch.Generator().manual_seed(7)).to(DEV)
    pos = torch.tensor([80, -1], dtype=torch.int64, device=DEV)
    y_plain = based.swa_decode_step(*dev(q, k, v), kc0, vc0, pos)
    y = base.clone()
    based.swa_decode_step(*dev(q, k, v), kc, vc, pos, add=y, y=y)
    assert torch.allclose(y[0], y_plain[0] + base[0], rtol=0, atol=1e-6)
    assert torch.isnan(y[1]).all() and torch.isnan(y_plain[1]).all()
    assert torch.equal(kc[1], kc0[1]) and torch.equal(vc[1], vc0[1])
    okc, ovc = oracle.swa_cache_fill(kp[:1], vp[:1], window)
    yo, _, _ = oracle.swa_decode_step(q[:1], k[:1], v[:1], okc, ovc, [80], window, 0.125)
    report("swa decode add (valid sequence)", ratio(y_plain[:1], yo), 2e-2)


def test_workload_window_decode_1p3b():
    """B=128, H=16, w=64 ring filled from a 104-token prefix, then 64 next-token
    steps; every step on 8 sampled heads is compared with the oracle's steps."""
    based = based_mod()
    wl = si.WORKLOADS["window_decode_1p3b"]
    _, k = si.window_inputs(wl)
    v = si.linear_inputs(wl)[2]
    kd, vd = dev(k, v)
    kc, vc = based.swa_cache_fill(kd, vd, window=wl.window)
    heads = _sample_heads(wl.B, wl.H, 8, 4)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    okc, ovc = oracle.swa_cache_fill(k[bi, hi][None], v[bi, hi][None], wl.window)
    pos = torch.full((wl.B,), wl.L, dtype=torch.int64, device=DEV)
    got, want = [], []
    for t in range(64):
        q1, k1, v1 = si.window_decode_inputs(wl, t)
        y = based.swa_decode_step(*dev(q1, k1, v1), kc, vc, pos, scale=wl.swa_scale)
        pos += 1
        got.append(y[bi, hi].cpu())
        yo, okc, ovc = oracle.swa_decode_step(q1[bi, hi][None], k1[bi, hi][None], v1[bi, hi][None], okc, ovc,
                                              [wl.L + t], wl.window, wl.swa_scale)
        want.append(yo[0])
    report("window_decode_1p3b (8 sampled heads, 64 steps)", ratio(torch.stack(got), np.stack(want)), wl.tol)


# ---------------------------------------------------------------- workloads
def test_workload_tiny_f32_layer():
    """B=1,H=1,L=256 fp32: Taylor linear attention + w=64 window, summed."""
    based = based_mod()
    wl = si.WORKLOADS["tiny_f32"]
    q, k, v = si.linear_inputs(wl)
    qd, kd, vd = dev(q, k, v)
    want = oracle.la_quadratic(q, k, v, eps=wl.eps) + oracle.swa(q, k, v, wl.window, wl.swa_scale)
    for chunk in (16, 32, 64):
        y, _, _ = based.based_prefill(qd, kd, vd, chunk=chunk, eps=wl.eps)
        based.swa_forward(qd, kd, vd, window=wl.window, scale=wl.swa_scale, add=y, y=y)
        report(f"tiny_f32 layer chunk={chunk}", ratio(y, want), wl.tol)


def _sample_heads(B, H, n, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(B * H, size=min(n, B * H), replace=False)
    return sorted((int(i) // H, int(i) % H) for i in idx)


def test_workload_prefill_360m():
    based = based_mod()
    wl = si.WORKLOADS["prefill_360m"]
    q, k, v = si.linear_inputs(wl)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    torch.cuda.synchronize()
    heads = _sample_heads(wl.B, wl.H, 16, 1)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    yo, So, zo = oracle.la_recurrent(q[bi, hi], k[bi, hi], v[bi, hi], eps=wl.eps)
    report("prefill_360m y (16 sampled heads)", ratio(y[bi, hi], yo), wl.tol)
    report("prefill_360m S (16 sampled heads)", ratio(S[bi, hi], So), wl.tol)


def test_workload_long_64k():
    based = based_mod()
    wl = si.WORKLOADS["long_64k"]
    q, k, v = si.linear_inputs(wl)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    torch.cuda.synchronize()
    hs = [3, 12]
    yo, So, zo = oracle.la_recurrent(q[0, hs], k[0, hs], v[0, hs], eps=wl.eps)
    report("long_64k y (2 sampled heads)", ratio(y[0, hs], yo), wl.tol)
    report("long_64k S (2 sampled heads)", ratio(S[0, hs], So), wl.tol)


# ---------------------------------------------------------------- hybrid layer
def _hybrid_inputs(B, H, L, seed, dqk=64, dtype=torch.bfloat16):
    q, k, v = si.custom((B, H, L, 16), (B, H, L, 64), seed=seed, scale=0.5, dtype=dtype)
    qw, kw, _ = si.custom((B, H, L, dqk), (1, 1, 1, 1), seed=seed + 10, scale=1.0, dtype=dtype)
    return q, k, v, qw, kw


@pytest.mark.parametrize("B,H,L", [(1, 2, 1), (2, 1, 33), (1, 2, 130), (2, 3, 257), (1, 2, 1000), (4, 64, 200)])
@pytest.mark.parametrize("window", [64, 17])
def test_hybrid_matches_oracle(B, H, L, window):
    """y = linear attention + window (each normalised on its own) in one
    pass, and the linear branch's final state.  The shapes cover one token,
    one chunk, a ragged tail, the segment split of few heads (the window's
    halo crosses every segment start) and the unsplit plan of many heads."""
    based = based_mod()
    q, k, v, qw, kw = _hybrid_inputs(B, H, L, seed=2400 + L + window + B)
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), window=window, scale=0.125, path="fused")
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v)
    want = yo + oracle.swa(qw, kw, v, window, 0.125)
    report(f"hybrid B={B} H={H} L={L} w={window} y", ratio(y, want), 2e-2)
    report(f"hybrid B={B} H={H} L={L} w={window} S", ratio(S, So), 2e-2)
    report(f"hybrid B={B} H={H} L={L} w={window} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("ws", ["auto", "none"])
def test_hybrid_initial_state(ws):
    """A carried linear-attention state (fused); with no workspace the fused
    kernel has no plan for two column groups, so "auto" runs the branches in
    turn and "fused" refuses."""
    based = based_mod()
    L = 300
    q, k, v, qw, kw = _hybrid_inputs(1, 3, L, seed=2450)
    qp, kp, vp = si.custom((1, 3, 50, 16), (1, 3, 50, 64), seed=2452, scale=0.5)
    _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
    S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
    kwargs = {"path": "fused"} if ws == "auto" else {"workspace": torch.empty(0, dtype=torch.uint8, device=DEV)}
    if ws == "none":
        with pytest.raises(based.BasedError):
            based.based_hybrid_prefill(*dev(q, k, qw, kw, v), initial_state=tuple(dev(S0, z0)), path="fused", **kwargs)
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), initial_state=tuple(dev(S0, z0)), **kwargs)
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    want = yo + oracle.swa(qw, kw, v, 64, 0.125)
    report(f"hybrid init-state ws={ws} y", ratio(y, want), 2e-2)
    report(f"hybrid init-state ws={ws} S", ratio(S, So), 2e-2)
    report(f"hybrid init-state ws={ws} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("dtype,tol,dqk,window", [
    (torch.bfloat16, 2e-2, 16, 64), (torch.bfloat16, 2e-2, 64, 100), (torch.float32, 1e-4, 64, 64),
])
def test_hybrid_composed_paths(dtype, tol, dqk, window):
    """Arguments without a fused kernel (16-dim window q/k, a window over
    64, fp32) run the two branches in turn; same result."""
    based = based_mod()
    q, k, v, qw, kw = _hybrid_inputs(1, 2, 200, seed=2460 + dqk + window, dqk=dqk, dtype=dtype)
    scale = dqk ** -0.5
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), window=window, scale=scale)
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"hybrid composed {dtype} dqk={dqk} w={window} y", ratio(y, yo + oracle.swa(qw, kw, v, window, scale)),
           tol)
    report(f"hybrid composed {dtype} dqk={dqk} w={window} S", ratio(S, So), tol)


def test_workload_window_8k_fused():
    """The 8K hybrid layer (B=4, H=16, L=8192) through the fused kernel, 3
    sampled heads against the oracle, and every element against the two
    branches run in turn (the same arithmetic up to rounding order)."""
    based = based_mod()
    wl = si.WORKLOADS["window_8k"]
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    qd, kd, vd, qwd, kwd = dev(q, k, v, qw, kw)
    y, S, z = based.based_hybrid_prefill(qd, kd, qwd, kwd, vd, chunk=wl.chunk, eps=wl.eps, window=wl.window,
                                         scale=wl.swa_scale, path="fused")
    y2, S2, z2 = based.based_prefill(qd, kd, vd, chunk=wl.chunk, eps=wl.eps)
    based.swa_forward(qwd, kwd, vd, window=wl.window, scale=wl.swa_scale, add=y2, y=y2)
    torch.cuda.synchronize()
    heads = _sample_heads(wl.B, wl.H, 3, 7)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    yo, So, zo = oracle.la_recurrent(q[bi, hi], k[bi, hi], v[bi, hi], eps=wl.eps)
    want = yo + oracle.swa(qw[bi, hi], kw[bi, hi], v[bi, hi], wl.window, wl.swa_scale)
    report("window_8k fused layer (3 sampled heads) y", ratio(y[bi, hi], want), wl.tol)
    report("window_8k fused layer (3 sampled heads) S", ratio(S[bi, hi], So), wl.tol)
    report("window_8k fused vs two passes (all heads)", float((y - y2).abs().max() / y2.pow(2).mean().sqrt()), wl.tol)


@pytest.mark.parametrize("B,H,L", [(8, 16, 256), (1, 2, 700)])
def test_hybrid_paths_agree(B, H, L):
    """auto, fused and two-pass give the same layer (rounding order aside),
    on a shape auto fuses (32-column plan) and one it does not fuse."""
    based = based_mod()
    q, k, v, qw, kw = _hybrid_inputs(B, H, L, seed=2480 + L)
    outs = {p: based.based_hybrid_prefill(*dev(q, k, qw, kw, v), scale=0.125, path=p)
            for p in ("auto", "fused", "two_pass")}
    torch.cuda.synchronize()
    ref = outs["two_pass"][0]
    rms = float(ref.pow(2).mean().sqrt())
    for p in ("auto", "fused"):
        report(f"hybrid {p} vs two-pass B={B} H={H} L={L}", float((outs[p][0] - ref).abs().max()) / rms, 2e-2)
        report(f"hybrid {p} vs two-pass S B={B} H={H} L={L}",
               float((outs[p][1] - outs["two_pass"][1]).abs().max() / outs["two_pass"][1].pow(2).mean().sqrt()), 2e-2)


def test_workload_window_8k():
    based = based_mod()
    wl = si.WORKLOADS["window_8k"]
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    qd, kd, vd, qwd, kwd = dev(q, k, v, qw, kw)
    y, _, _ = based.based_prefill(qd, kd, vd, chunk=wl.chunk, eps=wl.eps)
    based.swa_forward(qwd, kwd, vd, window=wl.window, scale=wl.swa_scale, add=y, y=y)
    torch.cuda.synchronize()
    heads = _sample_heads(wl.B, wl.H, 3, 2)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    want = oracle.la_recurrent(q[bi, hi], k[bi, hi], v[bi, hi], eps=wl.eps)[0] + oracle.swa(
        qw[bi, hi], kw[bi, hi], v[bi, hi], wl.window, wl.swa_scale)
    report("window_8k layer (3 sampled heads)", ratio(y[bi, hi], want), wl.tol)


def test_workload_decode_1p3b():
    """1024-token prefill then 1024 next-token steps; every step's output on
    8 sampled heads is compared, across all steps at once."""
    based = based_mod()
    wl = si.WORKLOADS["decode_1p3b"]
    q, k, v = si.linear_inputs(wl)
    _, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    heads = _sample_heads(wl.B, wl.H, 8, 3)
    bi = [b for b, _ in heads]
    hi = [h for _, h in heads]
    _, So, zo = oracle.la_recurrent(q[bi, hi], k[bi, hi], v[bi, hi], eps=wl.eps, want_y=False)
    got, want = [], []
    for t in range(wl.decode_steps):
        qt, kt, vt = si.decode_inputs(wl, t)
        y = based.based_decode_step(*dev(qt, kt, vt), S, z, eps=wl.eps)
        got.append(y[bi, hi].cpu())
        yo, So, zo = oracle.decode_step(qt[bi, hi], kt[bi, hi], vt[bi, hi], So, zo, eps=wl.eps)
        want.append(yo)
    report("decode_1p3b y (8 heads x 1024 steps)", ratio(torch.stack(got), np.stack(want)), wl.tol)
    report("decode_1p3b final S", ratio(S[bi, hi], So), wl.tol)
