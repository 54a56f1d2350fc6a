"""Host logic of bench.py, on the CPU: the algorithmic byte and flop counts
that the roofline fractions divide by, the reading of committed counter
summaries, and the one-GPU guard.

The expected counts are worked out here by hand from the quantities each
leg moves (bf16 q, k, v; fp32 y, state and normaliser; the 273-row Taylor
state of d' = 16), not from bench.py's formulas, so a dropped term or a
wrong element size there fails a test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synthetic_inputs as si  # noqa: E402

F = 1 + 16 + 16 * 16  # rows of the Taylor state for d' = 16
STATE_BYTES_64 = (F * 64 + F) * 4  # S and z of one head, d_v = 64, fp32


def test_prefill_bytes_headline():
    wl = si.WORKLOADS["prefill_360m"]
    # per token-head: q, k (16 bf16 each), v (64 bf16) read, y (64 fp32) written
    per_tok = 2 * 16 * 2 + 64 * 2 + 64 * 4
    assert per_tok == 448
    assert STATE_BYTES_64 == 70980
    assert bench.prefill_bytes(wl) == 8 * 16 * 2048 * 448 + 8 * 16 * 70980 == 126525952


def test_prefill_bytes_long_and_window_branch():
    assert bench.prefill_bytes(si.WORKLOADS["long_64k"]) == 16 * 65536 * 448 + 16 * 70980 == 470897728
    assert bench.prefill_bytes(si.WORKLOADS["window_8k"]) == 4 * 16 * 8192 * 448 + 64 * 70980 == 239423744


def test_prefill_bytes_fp32_inputs():
    wl = si.WORKLOADS["tiny_f32"]
    assert bench.prefill_bytes(wl) == 256 * (2 * 16 * 4 + 64 * 4 + 64 * 4) + 70980


def test_prefill_flops_headline():
    wl = si.WORKLOADS["prefill_360m"]
    # state update and readout: 2 flop per multiply-add over F x d_v each;
    # the causal on-diagonal term over the 65 (q.k, then weights.v) positions
    per_tok = 2 * (2 * F * 64) + 65 * (16 + 64)
    assert per_tok == 75088
    assert bench.prefill_flops(wl) == 8 * 16 * 2048 * 75088
    assert abs(bench.prefill_flops(wl) / 1e9 - 19.68) < 0.01


def test_setup_prefill_dv128():
    wl = si.WORKLOADS["decode_1p3b"]
    per_tok = 2 * 16 * 2 + 128 * 2 + 128 * 4
    assert per_tok == 832
    state = (F * 128 + F) * 4
    assert bench.prefill_bytes(wl) == 128 * 16 * 1024 * 832 + 128 * 16 * state == 2033328128
    assert bench.prefill_flops(wl) == 128 * 16 * 1024 * 149136


def test_decode_bytes():
    wl = si.WORKLOADS["decode_1p3b"]
    # S and z read and written back, q, k, v read (bf16), y written (fp32)
    per_head = 2 * F * 128 * 4 + 2 * F * 4 + 2 * 16 * 2 + 128 * 2 + 128 * 4
    assert per_head == 282568
    assert bench.decode_bytes(wl) == 128 * 16 * 282568 == 578699264


def test_window_bytes():
    wl = si.WORKLOADS["window_8k"]
    # q, k (64 bf16 each), v (64 bf16), add-in (64 fp32) read; y (64 fp32) written
    per_tok = 3 * 64 * 2 + 64 * 4 + 64 * 4
    assert per_tok == 896
    assert bench.swa_bytes(wl) == 4 * 16 * 8192 * 896 == 469762048


def test_hybrid_bytes():
    wl = si.WORKLOADS["window_8k"]
    # both branches' q and k (16 and 64 wide), the shared v read once, y written once
    per_tok = 2 * 16 * 2 + 2 * 64 * 2 + 64 * 2 + 64 * 4
    assert bench.hybrid_bytes(wl) == 4 * 16 * 8192 * per_tok + 64 * 70980


def test_window_decode_bytes():
    wl = si.WORKLOADS["window_decode_1p3b"]
    row = (64 + 128) * 2  # one cached key and value row, bf16
    # 63 older rows read, the new row written, q, k, v read, add-in read, y written
    per_head = 63 * row + row + (64 + 64 + 128) * 2 + 128 * 4 + 128 * 4
    assert per_head == 26112
    assert bench.window_decode_bytes(wl) == 128 * 16 * 26112 == 53477376


def test_backward_counts():
    wl = si.WORKLOADS["prefill_360m"]
    # q, k, v (bf16) and dy (fp32) read; dq, dk, dv (fp32) written
    per_tok = (16 + 16 + 64) * 2 + 64 * 4 + (16 + 16 + 64) * 4
    assert bench.backward_bytes(wl) == 8 * 16 * 2048 * per_tok
    n_pairs = 2048 * 2049 // 2
    per_pair = 8 * 16 + 6 * 64 + 12
    assert bench.backward_flops(wl, "direct") == 8 * 16 * n_pairs * per_pair
    sym = 1 + 16 + 16 * 17 // 2
    assert sym == 153
    chunked = 8 * 16 * 2048 * (6 * 2 * sym * 64 + 65 / 2 * per_pair)
    assert bench.backward_flops(wl, "chunked") == pytest.approx(chunked, rel=1e-12)


def test_window_backward_counts():
    wl = si.WORKLOADS["window_8k"]
    # q, k (64 bf16 each), v (64 bf16) and dy (64 fp32) read; dq, dk (64 fp32 each), dv (64 fp32) written
    per_tok = (64 + 64 + 64) * 2 + 64 * 4 + (64 + 64 + 64) * 4
    assert per_tok == 1408
    assert bench.swa_backward_bytes(wl) == 4 * 16 * 8192 * 1408
    # window-exact pairs: 1 + 2 + ... + 64 for the first 64 queries, then 64 each
    pairs = 64 * 65 // 2 + (8192 - 64) * 64
    assert bench.swa_backward_flops(wl) == 4 * 16 * pairs * (6 * 64 + 4 * 64)


def test_read_traffic(tmp_path):
    p = tmp_path / "summary.txt"
    p.write_text("# a comment: with a colon\n"
                 "kernel_source_sha256_16: 0123456789abcdef\n"
                 "hbm_bytes_per_launch: 126600000\n")
    assert bench.read_traffic(str(p), "0123456789abcdef") == 126600000.0
    # counters taken on another kernel source are not reported
    assert bench.read_traffic(str(p), "fedcba9876543210") is None
    assert bench.read_traffic(str(tmp_path / "absent.txt"), "0123456789abcdef") is None
    q = tmp_path / "bad.txt"
    q.write_text("kernel_source_sha256_16: 0123456789abcdef\nhbm_bytes_per_launch: n/a\n")
    assert bench.read_traffic(str(q), "0123456789abcdef") is None


def test_committed_summaries_are_readable():
    """Every committed counter summary names its source digest and a byte
    count; the digest is 16 hex digits as source_digest writes them."""
    names = [n for n in os.listdir(bench.PROFILES) if n.endswith("_pmc.txt")]
    assert names
    for n in names:
        vals = {}
        for line in open(os.path.join(bench.PROFILES, n)):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                vals[key.strip()] = val.strip()
        digest = vals.get("kernel_source_sha256_16", "")
        assert len(digest) == 16 and all(c in "0123456789abcdef" for c in digest), n
        assert bench.read_traffic(n, digest) == float(vals["hbm_bytes_per_launch"]) > 0, n


def test_every_gradient_leg_has_a_summary():
    """Each gradient leg that bench.py can profile has a committed counter
    summary under the name the bench reads, and the window gradients too."""
    for wname, form in bench.BACKWARD_PROFILE_LEGS.values():
        n = bench.backward_summary(wname, form)
        assert os.path.exists(os.path.join(bench.PROFILES, n)), n
    assert os.path.exists(os.path.join(bench.PROFILES, "swa_backward_window_8k_pmc.txt"))
    assert bench.backward_summary("prefill_360m", "chunked") == "prefill_backward_mfma_backward_360m_pmc.txt"


def test_source_digest_shape():
    d = bench.source_digest("prefill_mfma.hip")
    assert len(d) == 16 and d != bench.source_digest("decode.hip")


def test_more_than_one_gpu_is_refused():
    """--gpus 2 ends with status 2 and says why, before the library or the
    GPU is touched (so it runs here, without one)."""
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, env=env, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
