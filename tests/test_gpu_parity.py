"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.

Bar (max-abs error as a multiple of the oracle output's RMS over the whole
output tensor of the call): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
Full-size workloads are run on the GPU exactly as the benchmark launches
them and every element of every output is compared; where the oracle's
output would not fit in host memory at once, it is computed in blocks of
(batch, head) pairs (each pair is independent) and the maximum error and the
sum of squares are accumulated over the blocks.
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


class Streamed:
    """max |got - want| and the RMS of want over a tensor compared block by block."""

    def __init__(self):
        self.max_err, self.sumsq, self.n = 0.0, 0.0, 0

    def add(self, got, want):
        got = np.asarray(got.detach().cpu().double() if isinstance(got, torch.Tensor) else got, np.float64)
        want = np.asarray(want, np.float64)
        assert got.shape == want.shape, (got.shape, want.shape)
        self.max_err = max(self.max_err, float(np.abs(got - want).max()))
        self.sumsq += float(np.sum(want ** 2))
        self.n += want.size

    def ratio(self):
        return self.max_err / float(np.sqrt(self.sumsq / self.n))


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


@pytest.mark.parametrize("B,H,L,d,dtype,tol,dv,init", [
    (1, 2, 2048, 32, torch.float32, 1e-4, 64, False),   # 4 segments of 8 chunks
    (1, 1, 1500, 8, torch.bfloat16, 2e-2, 128, True),   # 2 segments, ragged tail
    (2, 3, 1100, 24, torch.float32, 1e-4, 64, True),    # 2 segments, ragged tail
    (1, 2, 1030, 16, torch.float32, 1e-4, 128, False),  # 9 + 8 chunks, the last one 6 tokens
])
def test_prefill_fp32_path_segments(B, H, L, d, dtype, tol, dv, init):
    """The fp32 matrix-core prefill split into sequence segments (few heads,
    long sequences): a state-only pass per segment, the prefix over
    segments from the caller's (asymmetric) initial state, and the output
    pass from the carried-in states.  y, S and z of every head against the
    oracle, with the default workspace and with none (one segment per
    head)."""
    based = based_mod()
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=780 + d + L, scale=0.5, dtype=dtype)
    kw, S0, z0 = {}, None, None
    if init:
        qp, kp, vp = si.custom((B, H, 40, d), (B, H, 40, dv), seed=782 + d, scale=0.5)
        _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
        S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
        P = torch.randn((B, H, d, d, dv), generator=torch.Generator().manual_seed(783 + d))
        S0[:, :, 1 + d:] += 0.5 * (P - P.transpose(2, 3)).reshape(B, H, d * d, dv)
    assert based.based_prefill_workspace_bytes(B, H, L, dv, d) > 0, "shape expected to split"
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    for ws in ("auto", "none"):
        if init:
            kw["initial_state"] = tuple(dev(S0, z0))
        if ws == "none":
            kw["workspace"] = torch.empty(0, dtype=torch.uint8, device=DEV)
        y, S, z = based.based_prefill(*dev(q, k, v), **kw)
        torch.cuda.synchronize()
        name = f"fp32-path segments {dtype} d={d} L={L} dv={dv} init={init} ws={ws}"
        report(f"{name} y", ratio(y, yo), tol)
        report(f"{name} S", ratio(S, So), tol)
        report(f"{name} z", ratio(z, zo), tol)


@pytest.mark.parametrize("dtype,tol,d", [(torch.float32, 1e-4, 16), (torch.bfloat16, 2e-2, 8)])
def test_prefill_fp32_path_resume_many_groups(dtype, tol, d):
    """The fp32 matrix-core prefill resuming from a carried state with far
    more workgroups (512 heads x 8 groups of 16 value columns) than are
    resident at once: every group must see the caller's initial z, however
    late it starts, and the final z must be the initial one plus this call's
    increment.  y, S and z of every head against the oracle."""
    based = based_mod()
    B, H, L, dv = 8, 64, 300, 128
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=770 + d, scale=0.5, dtype=dtype)
    qp, kp, vp = si.custom((B, H, 40, d), (B, H, 40, dv), seed=772 + d, scale=0.5)
    _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
    S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
    y, S, z = based.based_prefill(*dev(q, k, v), initial_state=tuple(dev(S0, z0)))
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    report(f"fp32-path resume, many groups {dtype} d={d} y", ratio(y, yo), tol)
    report(f"fp32-path resume, many groups {dtype} d={d} S", ratio(S, So), tol)
    report(f"fp32-path resume, many groups {dtype} d={d} z", ratio(z, zo), tol)


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
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"many-heads dv={dv} y", ratio(y, yo), 2e-2)
    report(f"many-heads dv={dv} S", ratio(S, So), 2e-2)
    report(f"many-heads dv={dv} z", ratio(z, zo), 2e-2)


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


@pytest.mark.parametrize("L,H,d,dtype", [(300, 2, 16, torch.bfloat16), (2048, 4, 16, torch.bfloat16),
                                         (2048, 2, 8, torch.bfloat16), (1500, 2, 16, torch.float32)])
def test_prefill_graph_replay(L, H, d, dtype):
    """Captured in a HIP graph (as the benchmark runs it), every replay gives
    the eager result bit for bit, with eager work and synchronisation in
    between replays.  (2048, 4) takes the segment split of the bf16 matrix
    cores and its workspace; d' = 8 and the fp32 inputs, the segment split
    of the fp32 matrix-core path (state-only pass, prefix, output pass)."""
    based = based_mod()
    F = 1 + d + d * d
    q, k, v = dev(*si.custom((1, H, L, d), (1, H, L, 64), seed=810 + L, scale=0.5, dtype=dtype))
    nbytes = based.based_prefill_workspace_bytes(1, H, L, 64, d)
    assert L < 1024 or nbytes > 0
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty(1, H, L, 64, device=DEV)
    S = torch.empty(1, H, F, 64, device=DEV)
    z = torch.empty(1, H, F, device=DEV)
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


def _replay_matches(g, outs, ref, reset=None, eager=None):
    """Replay g three times: before each replay the outputs are poisoned
    (and `reset` restores in-place state); after it every output must equal
    the eager result bit for bit; eager work runs in between."""
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        if reset:
            reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outs, ref)):
            assert torch.equal(got, want), f"replay {rep}: output {i} differs from the eager result"
        if eager:
            eager()
        torch.cuda.synchronize()


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up off the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_hybrid_and_backward_graph_replay():
    """The multi-launch calls under HIP graph capture: the hybrid layer on
    its segment plan (state pass, prefix, fused segment pass) and the
    chunked gradients (segment sums, query sweep, key sweep), each with a
    caller workspace; every replay equals the eager result bit for bit."""
    based = based_mod()
    B, H, L = 1, 4, 2048
    q, k, v, qw, kw = dev(*_hybrid_inputs(B, H, L, seed=3100))
    F = 1 + 16 + 16 * 16
    y, S, z = (torch.empty(B, H, L, 64, device=DEV), torch.empty(B, H, F, 64, device=DEV),
               torch.empty(B, H, F, device=DEV))
    wsh = torch.empty(max(1, based.based_hybrid_prefill_workspace_bytes(B, H, L, 64)), dtype=torch.uint8, device=DEV)
    run_h = lambda: based.based_hybrid_prefill(q, k, qw, kw, v, window=64, scale=0.125, y=y, S=S, z=z,  # noqa: E731
                                               workspace=wsh)
    ref = [t.clone() for t in run_h()]
    _replay_matches(_capture(run_h), (y, S, z), ref, eager=lambda: based.based_prefill(q[:, :1], k[:, :1], v[:, :1]))

    dy = torch.randn(B, H, L, 64, generator=torch.Generator().manual_seed(3101)).to(DEV)
    dq, dk, dv = (torch.empty(B, H, L, 16, device=DEV), torch.empty(B, H, L, 16, device=DEV),
                  torch.empty(B, H, L, 64, device=DEV))
    wsb = torch.empty(based.based_prefill_backward_workspace_bytes(B, H, L, 64), dtype=torch.uint8, device=DEV)
    run_b = lambda: based.based_prefill_backward(q, k, v, dy, form="chunked", dq=dq, dk=dk, dv=dv,  # noqa: E731
                                                 workspace=wsb)
    ref = [t.clone() for t in run_b()]
    _replay_matches(_capture(run_b), (dq, dk, dv), ref, eager=lambda: based.based_prefill(q[:, :1], k[:, :1], v[:, :1]))


def test_layer_step_graph_replay():
    """One layer's next-token step under HIP graph capture: the linear
    decode step (state updated in place, restored before each replay) and
    the window step adding into its output (ring cache updated in place, the
    same slot each replay)."""
    based = based_mod()
    B, H, L, window = 4, 8, 100, 64
    q, k, v, qw, kw = dev(*_hybrid_inputs(B, H, L + 1, seed=3200))
    _, S, z = based.based_prefill(q[:, :, :L].contiguous(), k[:, :, :L].contiguous(), v[:, :, :L].contiguous())
    kc, vc = based.swa_cache_fill(kw[:, :, :L].contiguous(), v[:, :, :L].contiguous(), window=window)
    S0, z0 = S.clone(), z.clone()
    qt, kt, vt = (x[:, :, L].contiguous() for x in (q, k, v))
    qwt, kwt = (x[:, :, L].contiguous() for x in (qw, kw))
    pos = torch.full((B,), L, dtype=torch.int64, device=DEV)
    y_la = torch.empty(B, H, 64, device=DEV)
    y = torch.empty(B, H, 64, device=DEV)

    def step():
        based.based_decode_step(qt, kt, vt, S, z, y=y_la)
        based.swa_decode_step(qwt, kwt, vt, kc, vc, pos, scale=0.125, add=y_la, y=y)

    def reset():
        S.copy_(S0)
        z.copy_(z0)

    step()
    ref = [y.clone(), S.clone(), z.clone()]
    g = _capture(step)  # the state is restored eagerly before each replay
    _replay_matches(g, (y,), ref[:1], reset=reset)
    assert torch.equal(S, ref[1]) and torch.equal(z, ref[2])


def test_prefill_deterministic():
    based = based_mod()
    q, k, v = dev(*si.custom((2, 2, 300, 16), (2, 2, 300, 64), seed=800, scale=0.5))
    a = [t.clone() for t in based.based_prefill(q, k, v)]
    b = based.based_prefill(q, k, v)
    for x, w in zip(a, b):
        assert torch.equal(x, w)


@pytest.mark.parametrize("H,L,d,dtype,tol", [
    (2, 4096, 16, torch.bfloat16, 2e-2),  # bf16 matrix cores, segment split
    (2, 2048, 32, torch.float32, 1e-4),   # fp32 matrix cores, segment split
    (3, 333, 8, torch.bfloat16, 2e-2),    # fp32 matrix cores, one segment
])
def test_prefill_zero_queries_running_mean(H, L, d, dtype, tol):
    """Closed form, independent of the oracle: with q = 0 every weight
    phi(q).phi(k) is 1, so y_i = (sum_{j<=i} v_j) / (i + 1 + eps), a causal
    running mean, whatever the keys; the final z is sum_j phi(k_j) and
    S = sum_j phi(k_j) v_j^T, whose constant row is sum_j v_j and count
    row z_0 = L."""
    based = based_mod()
    _, k, v = si.custom((1, H, L, d), (1, H, L, 64), seed=820 + d, scale=0.5, dtype=dtype)
    q = torch.zeros_like(k)
    y, S, z = based.based_prefill(*dev(q, k, v))
    torch.cuda.synchronize()
    vd = v.double()
    cnt = torch.arange(1, L + 1, dtype=torch.float64).view(1, 1, L, 1)
    want = vd.cumsum(2) / (cnt + 1e-6)
    report(f"zero queries d={d} {dtype} L={L}: y vs running mean", ratio(y, want.numpy()), tol)
    report(f"zero queries d={d} {dtype} L={L}: S constant row vs sum of v", ratio(S[:, :, 0], vd.sum(2).numpy()), tol)
    assert torch.allclose(z[:, :, 0].double().cpu(), torch.full((1, H), float(L), dtype=torch.float64), rtol=1e-6)


@pytest.mark.parametrize("window,dtype,tol,dv", [(64, torch.bfloat16, 2e-2, 64), (64, torch.float32, 1e-4, 128),
                                                 (129, torch.bfloat16, 2e-2, 128), (7, torch.bfloat16, 2e-2, 64)])
def test_swa_zero_queries_window_mean(window, dtype, tol, dv):
    """Closed form, independent of the oracle: with q = 0 every logit is 0,
    so y_i is the plain mean of the last min(i + 1, w) values."""
    based = based_mod()
    B, H, L = 1, 3, 700
    _, k, v = si.custom((B, H, L, 64), (B, H, L, dv), seed=830 + window, scale=1.0, dtype=dtype)
    q = torch.zeros_like(k)
    y = based.swa_forward(*dev(q, k, v), window=window, scale=0.125)
    torch.cuda.synchronize()
    c = torch.cat([torch.zeros(B, H, 1, dv, dtype=torch.float64), v.double().cumsum(2)], dim=2)
    i = torch.arange(L)
    j0 = (i - window + 1).clamp(min=0)
    want = (c[:, :, i + 1] - c[:, :, j0]) / (i - j0 + 1).double().view(1, 1, L, 1)
    report(f"window zero queries w={window} {dtype} dv={dv}: y vs window mean", ratio(y, want.numpy()), tol)


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
    want = oracle.swa(q, k, v, window, scale)
    if add:
        want = want + base.double().numpy()
    report(f"swa long runs dqk={dqk} add={add} w={window} (all heads)", ratio(outs[0], want), 2e-2)


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


@pytest.mark.parametrize("dtype,tol", [(torch.bfloat16, 2e-2), (torch.float32, 1e-4)])
@pytest.mark.parametrize("dqk", [16, 64])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("window,L", [(1, 70), (64, 200), (129, 300), (256, 700), (700, 700), (10**9, 900),
                                      (128, 1)])
def test_swa_any_window_width(dtype, tol, dqk, dv, window, L):
    """Every window (1, 64, over 128 keys, the whole causal prefix, one far
    beyond the sequence) at 64 and 128 value columns, with a fused add."""
    based = based_mod()
    q, k, v = si.custom((1, 3, L, dqk), (1, 3, L, dv), seed=1950 + window % 1000 + L + dqk + dv, scale=1.0,
                        dtype=dtype)
    base = torch.randn(1, 3, L, dv, generator=torch.Generator().manual_seed(1951))
    scale = dqk ** -0.5
    y = based.swa_forward(*dev(q, k, v), window=window, scale=scale, add=base.to(DEV))
    want = oracle.swa(q, k, v, window, scale) + base.double().numpy()
    report(f"swa {dtype} dqk={dqk} dv={dv} w={window} L={L}", ratio(y, want), tol)


def test_swa_full_causal_many_heads():
    """w >= L (plain causal softmax attention) over B*H = 48 heads, d_v =
    128: many workgroups, the longest key ranges scheduled first; every
    element against the oracle."""
    based = based_mod()
    q, k, v = si.custom((4, 12, 1500, 64), (4, 12, 1500, 128), seed=1960, scale=1.0)
    y = based.swa_forward(*dev(q, k, v), window=1500, scale=0.125)
    report("swa full causal 48 heads dv=128", ratio(y, oracle.swa(q, k, v, 1500, 0.125)), 2e-2)


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


@pytest.mark.parametrize("B,H,L", [(1, 2, 3), (1, 1, 64), (2, 1, 65), (1, 2, 130), (1, 3, 257), (2, 2, 700),
                                   (2, 4, 4100)])
def test_backward_chunked_matches_oracle(B, H, L):
    """The chunked (linear-time) form, bf16 with d' = 16 and d_v = 64: every
    element of dq, dk, dv against the oracle.  The shapes span one chunk,
    ragged tails, one segment per chunk, and (8 heads of 4100 tokens)
    segments of two chunks ending in a one-chunk segment."""
    based = based_mod()
    q, k, v = si.custom((B, H, L, 16), (B, H, L, 64), seed=2400 + L + H, scale=0.5)
    dy = torch.randn(B, H, L, 64, generator=torch.Generator().manual_seed(2401 + L))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), form="chunked")
    torch.cuda.synchronize()
    want = oracle.la_backward(q, k, v, dy) if L <= 1000 else oracle.la_backward_recurrent(q, k, v, dy)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv_), want):
        report(f"chunked backward B={B} H={H} L={L} {name}", ratio(got, w), 2e-2)


@pytest.mark.parametrize("B,H,L", [(1, 2, 3), (2, 1, 65), (1, 3, 257), (2, 2, 700), (2, 4, 4100)])
def test_backward_chunked_dv128_matches_oracle(B, H, L):
    """The chunked form at d_v = 128 (one pass per 64-column half, the second
    adding into dq and dk): every element of dq, dk, dv against the oracle,
    at one chunk, ragged tails and segmented heads."""
    based = based_mod()
    q, k, v = si.custom((B, H, L, 16), (B, H, L, 128), seed=2450 + L + H, scale=0.5)
    dy = torch.randn(B, H, L, 128, generator=torch.Generator().manual_seed(2451 + L))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), form="chunked")
    torch.cuda.synchronize()
    want = oracle.la_backward(q, k, v, dy) if L <= 1000 else oracle.la_backward_recurrent(q, k, v, dy)
    for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv_), want):
        report(f"chunked backward d_v=128 B={B} H={H} L={L} {name}", ratio(got, w), 2e-2)


@pytest.mark.parametrize("form", ["direct", "chunked"])
@pytest.mark.parametrize("dvd", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_backward_single_token(dtype, dvd, form):
    """L = 1: y_0 = v_0 a/(a + eps), so dv_0 = dy_0 a/(a + eps) and dq, dk are
    of order eps: they come out of the cancellation of terms of order
    |dy||v|, and fp32 gives them to rounding noise of those terms."""
    if form == "chunked" and dtype != torch.bfloat16:
        pytest.skip("the chunked form takes bf16 inputs")
    based = based_mod()
    q, k, v = si.custom((2, 2, 1, 16), (2, 2, 1, dvd), seed=2250, scale=1.0, dtype=dtype)
    dy = torch.randn(2, 2, 1, dvd, generator=torch.Generator().manual_seed(2251))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), form=form)
    oq, ok, ov = oracle.la_backward(q, k, v, dy)
    report(f"backward L=1 {dtype} d_v={dvd} {form} dv", ratio(dv_, ov), 1e-4)
    noise = 1e-5 * float(dy.norm(dim=-1).max() * v.float().norm(dim=-1).max() * k.float().norm(dim=-1).max())
    assert float(dq.abs().max()) <= noise and float(dk.abs().max()) <= noise, (dq.abs().max(), dk.abs().max(), noise)
    assert np.abs(oq).max() <= noise and np.abs(ok).max() <= noise


def test_workload_prefill_360m_backward():
    """Gradients over the 360M-shaped layer (B=8, H=16, L=2048): dq, dk, dv
    of all 128 heads in both forms (chunked: segments of 8 chunks) against
    the oracle's chain rule."""
    based = based_mod()
    wl = si.WORKLOADS["prefill_360m"]
    q, k, v = si.linear_inputs(wl)
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2300))
    oq, ok, ov = oracle.la_backward(q, k, v, dy, eps=wl.eps)
    for form in ("direct", "chunked"):
        dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), eps=wl.eps, form=form)
        torch.cuda.synchronize()
        report(f"prefill_360m backward {form} dq (all heads)", ratio(dq, oq), wl.tol)
        report(f"prefill_360m backward {form} dk (all heads)", ratio(dk, ok), wl.tol)
        report(f"prefill_360m backward {form} dv (all heads)", ratio(dv_, ov), wl.tol)
        del dq, dk, dv_


def test_workload_1p3b_backward_sampled_heads():
    """Gradients over the 1.3B-shaped layer (B=128, H=16, L=1024, d_v=128)
    in both forms (the chunked one as two column-half passes): dq, dk, dv
    of 8 seeded (batch, head) pairs against the oracle's chain rule on those
    heads alone (heads do not interact), and every output finite."""
    based = based_mod()
    wl = si.WORKLOADS["decode_1p3b"]
    q, k, v = si.linear_inputs(wl)
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2320))
    rng = np.random.default_rng(2321)
    picks = [(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(8)]
    sel = lambda x: torch.stack([x[b, h] for b, h in picks])[None]
    oq, ok, ov = oracle.la_backward(sel(q), sel(k), sel(v), sel(dy), eps=wl.eps)
    qd, kd, vd = dev(q, k, v)
    dyd = dy.to(DEV)
    for form in ("direct", "chunked"):
        print(f"[1p3b backward] form={form}", flush=True)
        dq, dk, dv_ = based.based_prefill_backward(qd, kd, vd, dyd, eps=wl.eps, form=form)
        torch.cuda.synchronize()
        for name, got, w in zip(("dq", "dk", "dv"), (dq, dk, dv_), (oq, ok, ov)):
            assert bool(torch.isfinite(got).all()), (form, name)
            report(f"decode_1p3b-shaped backward {form} {name} (8 heads)", ratio(sel(got.cpu()), w), wl.tol)
        del dq, dk, dv_


@pytest.mark.timeout(900)
def test_workload_long_64k_backward():
    """Gradients over the 64K sequence (B=1, H=16, L=65536, outlier keys)
    in the chunked form (segments of 32 chunks): every element of dq, dk,
    dv of all 16 heads against the oracle's recurrent-form gradients."""
    based = based_mod()
    wl = si.WORKLOADS["long_64k"]
    q, k, v = si.linear_inputs(wl)
    dy = torch.randn(wl.B, wl.H, wl.L, wl.dv, generator=torch.Generator().manual_seed(2350))
    dq, dk, dv_ = based.based_prefill_backward(*dev(q, k, v), dy.to(DEV), eps=wl.eps)
    torch.cuda.synchronize()
    oq, ok, ov = oracle.la_backward_recurrent(q, k, v, dy, eps=wl.eps)
    report("long_64k backward dq (all heads)", ratio(dq, oq), wl.tol)
    report("long_64k backward dk (all heads)", ratio(dk, ok), wl.tol)
    report("long_64k backward dv (all heads)", ratio(dv_, ov), wl.tol)


# ---------------------------------------------------------------- window decode
def _nan_cache(B, H, window, d, dtype):
    return torch.full((B, H, window, d), float("nan"), dtype=dtype, device=DEV)


@pytest.mark.parametrize("dtype,dqk,dv,window,L", [
    (torch.bfloat16, 64, 64, 64, 100), (torch.bfloat16, 16, 128, 64, 10), (torch.bfloat16, 64, 128, 7, 30),
    (torch.bfloat16, 64, 64, 64, 0), (torch.float32, 64, 64, 64, 64), (torch.float32, 16, 128, 1, 5),
    (torch.float32, 64, 128, 33, 200), (torch.bfloat16, 64, 128, 128, 200), (torch.float32, 16, 64, 100, 10),
    (torch.bfloat16, 64, 64, 128, 0),
    # windows over 128: the online-softmax kernel, one or several rounds per wave
    (torch.bfloat16, 64, 128, 129, 300), (torch.float32, 16, 64, 200, 10), (torch.bfloat16, 64, 64, 300, 0),
    (torch.float32, 64, 128, 257, 600), (torch.bfloat16, 16, 128, 600, 1500),
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


@pytest.mark.parametrize("window", [64, 300])
def test_swa_decode_add_and_invalid_position(window):
    """add (fused sum, in place on y); a negative position gives NaN outputs
    for its sequence and leaves that sequence's cache untouched (the
    one-wave kernel and, at w = 300, the workgroup-per-head kernel; the
    prefix is 16 tokens longer than the window, so the ring has wrapped)."""
    based = based_mod()
    B, H, P = 2, 2, window + 16
    q, k, v = si.custom((B, H, 64), (B, H, 64), seed=1700)
    kp, vp = si.custom((B, H, P, 64), (B, H, P, 64), seed=1701)[1:]
    kc, vc = based.swa_cache_fill(*dev(kp, vp), window=window)
    kc0, vc0 = kc.clone(), vc.clone()
    base = torch.randn(B, H, 64, generator=torch.Generator().manual_seed(7)).to(DEV)
    pos = torch.tensor([P, -1], dtype=torch.int64, device=DEV)
    y_plain = based.swa_decode_step(*dev(q, k, v), kc0, vc0, pos)
    y = base.clone()
    based.swa_decode_step(*dev(q, k, v), kc, vc, pos, add=y, y=y)
    assert torch.allclose(y[0], y_plain[0] + base[0], rtol=0, atol=1e-6)
    assert torch.isnan(y[1]).all() and torch.isnan(y_plain[1]).all()
    assert torch.equal(kc[1], kc0[1]) and torch.equal(vc[1], vc0[1])
    okc, ovc = oracle.swa_cache_fill(kp[:1], vp[:1], window)
    yo, _, _ = oracle.swa_decode_step(q[:1], k[:1], v[:1], okc, ovc, [P], window, 0.125)
    report(f"swa decode add w={window} (valid sequence)", ratio(y_plain[:1], yo), 2e-2)


@pytest.mark.timeout(600)
def test_workload_window_decode_1p3b():
    """B=128, H=16, w=64 ring filled from a 104-token prefix, then 1024
    next-token steps.  Every step's output for all 2048 heads is compared
    with the oracle's brute-force window attention over the whole sequence
    (prefix and step tokens; pin P8 ties the oracle's ring steps to it), and
    the final caches with the oracle's ring of the whole sequence, exactly."""
    based = based_mod()
    wl = si.WORKLOADS["window_decode_1p3b"]
    _, k = si.window_inputs(wl)
    v = si.linear_inputs(wl)[2]
    kc, vc = based.swa_cache_fill(*dev(k, v), window=wl.window)
    T = wl.decode_steps
    pos = torch.full((wl.B,), wl.L, dtype=torch.int64, device=DEV)
    steps = [si.window_decode_inputs(wl, t) for t in range(T)]
    ys = torch.empty((T, wl.B, wl.H, wl.dv), dtype=torch.float32, device=DEV)
    for t in range(T):
        based.swa_decode_step(*dev(*steps[t]), kc, vc, pos, scale=wl.swa_scale, y=ys[t])
        pos += 1
    torch.cuda.synchronize()
    qa = torch.stack([s_[0] for s_ in steps], dim=2)  # only the step tokens query
    ka = torch.cat([k, torch.stack([s_[1] for s_ in steps], dim=2)], dim=2)
    va = torch.cat([v, torch.stack([s_[2] for s_ in steps], dim=2)], dim=2)
    # queries of the prefix do not matter: run the oracle with zeros there
    qfull = torch.cat([torch.zeros_like(k), qa], dim=2)
    want = oracle.swa(qfull, ka, va, wl.window, wl.swa_scale)[:, :, wl.L:]
    report(f"window_decode_1p3b (all heads, {T} steps)", ratio(ys.permute(1, 2, 0, 3), want), wl.tol)
    okc, ovc = oracle.swa_cache_fill(ka, va, wl.window)
    np.testing.assert_array_equal(kc.double().cpu().numpy(), okc)
    np.testing.assert_array_equal(vc.double().cpu().numpy(), ovc)


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


def test_workload_prefill_360m():
    """The 360M-shaped layer (B=8, H=16, L=2048): y, S and z of all 128
    heads against the oracle's recurrent form."""
    based = based_mod()
    wl = si.WORKLOADS["prefill_360m"]
    q, k, v = si.linear_inputs(wl)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, eps=wl.eps)
    report("prefill_360m y (all heads)", ratio(y, yo), wl.tol)
    report("prefill_360m S (all heads)", ratio(S, So), wl.tol)
    report("prefill_360m z (all heads)", ratio(z, zo), wl.tol)


def test_workload_long_64k():
    """The 64K sequence (B=1, H=16, L=65536, outlier keys), segment split:
    every element of y, S, z of all 16 heads."""
    based = based_mod()
    wl = si.WORKLOADS["long_64k"]
    q, k, v = si.linear_inputs(wl)
    y, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, eps=wl.eps)
    report("long_64k y (all heads)", ratio(y, yo), wl.tol)
    report("long_64k S (all heads)", ratio(S, So), wl.tol)
    report("long_64k z (all heads)", ratio(z, zo), wl.tol)


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


@pytest.mark.parametrize("L1,T,window", [(200, 24, 64), (37, 40, 64), (130, 16, 17)])
def test_hybrid_prefill_then_layer_steps(L1, T, window):
    """The serving path of one layer ("Simple linear attention language
    models balance the recall-throughput tradeoff", App. B, Forward /
    Generation Prefill then Next Token Prediction): based_hybrid_prefill
    over the first L1 tokens, then swa_cache_fill of the window's ring, then
    T per-token layer steps (based_decode_step on the prefill's state, and
    swa_decode_step adding into its output).  Every output row, of the
    prefill and of the steps, is compared with the oracle run over the whole
    L1 + T tokens (linear attention plus the window, each normalised on its
    own), and so is the state after the last step."""
    based = based_mod()
    B, H, L = 2, 3, L1 + T
    q, k, v, qw, kw = _hybrid_inputs(B, H, L, seed=2900 + L1 + T + window)
    scale = 0.125
    yo, So, zo = oracle.la_recurrent(q, k, v)
    want = yo + oracle.swa(qw, kw, v, window, scale)
    qd, kd, vd, qwd, kwd = dev(q, k, v, qw, kw)
    pre = [x[:, :, :L1].contiguous() for x in (qd, kd, qwd, kwd, vd)]
    y1, S, z = based.based_hybrid_prefill(*pre, window=window, scale=scale)
    kc, vc = based.swa_cache_fill(pre[3], pre[4], window=window)
    steps = []
    for t in range(L1, L):
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        y_la = based.based_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                       S, z)
        steps.append(based.swa_decode_step(qwd[:, :, t].contiguous(), kwd[:, :, t].contiguous(),
                                           vd[:, :, t].contiguous(), kc, vc, pos, scale=scale, add=y_la))
    torch.cuda.synchronize()
    got = torch.cat([y1.cpu(), torch.stack([y.cpu() for y in steps], dim=2)], dim=2)
    report(f"hybrid prefill {L1} + {T} layer steps w={window} y", ratio(got, want), 2e-2)
    report(f"hybrid prefill {L1} + {T} layer steps w={window} S", ratio(S, So), 2e-2)
    report(f"hybrid prefill {L1} + {T} layer steps w={window} z", ratio(z, zo), 2e-2)


@pytest.mark.parametrize("B,H,L", [(1, 2, 1), (2, 1, 37), (1, 3, 130), (2, 2, 333)])
@pytest.mark.parametrize("window", [64, 17, 1])
@pytest.mark.parametrize("dv", [64, 128])
def test_swa_backward_matches_oracle(B, H, L, window, dv):
    """Gradients of the window (bf16, d_qk = 64) against the oracle's chain
    rule through the softmax: one token, ragged tails, one and several
    64-row tiles, windows of 64, 17 and 1 keys (w = 1: dq = dk = 0,
    dv = dy)."""
    based = based_mod()
    q, k, v = si.custom((B, H, L, 64), (B, H, L, dv), seed=3300 + L + window + dv, scale=1.0)
    dy = torch.randn(B, H, L, dv, generator=torch.Generator().manual_seed(3301 + L))
    a = based.swa_backward(*dev(q, k, v, dy), window=window, scale=0.125)
    b = based.swa_backward(*dev(q, k, v, dy), window=window, scale=0.125)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    want = oracle.swa_backward(q, k, v, dy, window, 0.125)
    for name, got, w in zip(("dq", "dk", "dv"), a, want):
        if not np.any(w):
            assert not torch.any(got), name  # w = 1: exactly zero
            continue
        report(f"swa backward B={B} H={H} L={L} w={window} dv={dv} {name}", ratio(got, w), 2e-2)


def test_swa_backward_window_8k_heads():
    """The 8K layer's window branch (L = 8192, d_qk = d_v = 64, w = 64) on
    four heads, every element against the oracle."""
    based = based_mod()
    wl = si.WORKLOADS["window_8k"]
    _, _, v = si.linear_inputs(wl, B=1, H=4)
    q, k = si.window_inputs(wl, B=1, H=4)
    dy = torch.randn(1, 4, wl.L, wl.dv, generator=torch.Generator().manual_seed(3302))
    got = based.swa_backward(*dev(q, k, v, dy), window=wl.window, scale=wl.swa_scale)
    torch.cuda.synchronize()
    want = oracle.swa_backward(q, k, v, dy, wl.window, wl.swa_scale)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        report(f"swa backward 8K layer (4 heads) {name}", ratio(g, w), 2e-2)


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


@pytest.mark.parametrize("dtype,tol,dqk,window,L", [
    (torch.bfloat16, 2e-2, 16, 64, 200), (torch.bfloat16, 2e-2, 64, 100, 200), (torch.float32, 1e-4, 64, 64, 200),
    (torch.float32, 1e-4, 64, 64, 2100),  # the linear branch split into segments (fp32 matrix cores)
])
def test_hybrid_composed_paths(dtype, tol, dqk, window, L):
    """Arguments without a fused kernel (16-dim window q/k, a window over
    64, fp32) run the two branches in turn; same result."""
    based = based_mod()
    q, k, v, qw, kw = _hybrid_inputs(1, 2, L, seed=2460 + dqk + window, dqk=dqk, dtype=dtype)
    scale = dqk ** -0.5
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), window=window, scale=scale)
    yo, So, zo = oracle.la_recurrent(q, k, v)
    report(f"hybrid composed {dtype} dqk={dqk} w={window} y", ratio(y, yo + oracle.swa(qw, kw, v, window, scale)),
           tol)
    report(f"hybrid composed {dtype} dqk={dqk} w={window} S", ratio(S, So), tol)


@pytest.mark.parametrize("path", ["fused", "two_pass"])
@pytest.mark.parametrize("B,H,L,window", [(1, 2, 130, 64), (2, 3, 1000, 64), (8, 16, 1024, 64), (1, 2, 300, 200)])
def test_hybrid_dv128(path, B, H, L, window):
    """Value width 128 (the 1.3B layer's), fused (four 32-column groups, the
    segment split for few heads) and as two passes; (8, 16, 1024) is the
    1.3B-shaped layer at a reduced batch.  A window over 64 keys has no
    fused kernel: "fused" must refuse it."""
    based = based_mod()
    q, k, _ = si.custom((B, H, L, 16), (1, 1, 1, 1), seed=2490 + L + B, scale=0.5)
    v = si.randn((B, H, L, 128), 2493 + L, 1.0, torch.bfloat16)
    qw, kw, _ = si.custom((B, H, L, 64), (1, 1, 1, 1), seed=2495 + L, scale=1.0)
    if path == "fused" and window > 64:
        with pytest.raises(based.BasedError):
            based.based_hybrid_prefill(*dev(q, k, qw, kw, v), window=window, scale=0.125, path=path)
        return
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), window=window, scale=0.125, path=path)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v)
    want = yo + oracle.swa(qw, kw, v, window, 0.125)
    report(f"hybrid dv=128 {path} B={B} H={H} L={L} w={window} y", ratio(y, want), 2e-2)
    report(f"hybrid dv=128 {path} B={B} H={H} L={L} w={window} S", ratio(S, So), 2e-2)
    report(f"hybrid dv=128 {path} B={B} H={H} L={L} w={window} z", ratio(z, zo), 2e-2)


def test_hybrid_dv128_initial_state():
    """d_v = 128, a carried state, fused (through the workspace)."""
    based = based_mod()
    L = 400
    q, k, _ = si.custom((1, 3, L, 16), (1, 1, 1, 1), seed=2497, scale=0.5)
    v = si.randn((1, 3, L, 128), 2498, 1.0, torch.bfloat16)
    qw, kw, _ = si.custom((1, 3, L, 64), (1, 1, 1, 1), seed=2499, scale=1.0)
    qp, kp, vp = si.custom((1, 3, 50, 16), (1, 3, 50, 128), seed=2500, scale=0.5)
    _, S0, z0 = oracle.la_recurrent(qp, kp, vp, want_y=False)
    S0, z0 = torch.as_tensor(S0, dtype=torch.float32), torch.as_tensor(z0, dtype=torch.float32)
    y, S, z = based.based_hybrid_prefill(*dev(q, k, qw, kw, v), initial_state=tuple(dev(S0, z0)), path="fused")
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    report("hybrid dv=128 init-state y", ratio(y, yo + oracle.swa(qw, kw, v, 64, 0.125)), 2e-2)
    report("hybrid dv=128 init-state S", ratio(S, So), 2e-2)
    report("hybrid dv=128 init-state z", ratio(z, zo), 2e-2)


def test_workload_window_8k_fused():
    """The 8K hybrid layer (B=4, H=16, L=8192) through the fused kernel:
    every element of y, S and z of all 64 heads against the oracle, and y
    against the two branches run in turn (the same arithmetic up to rounding
    order)."""
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
    yo, So, zo = oracle.la_recurrent(q, k, v, eps=wl.eps)
    want = yo + oracle.swa(qw, kw, v, wl.window, wl.swa_scale)
    report("window_8k fused layer y (all heads)", ratio(y, want), wl.tol)
    report("window_8k fused layer S (all heads)", ratio(S, So), wl.tol)
    report("window_8k fused layer z (all heads)", ratio(z, zo), wl.tol)
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
    """The 8K layer as two calls (linear attention, then the window adding
    into y in place): every element of all 64 heads."""
    based = based_mod()
    wl = si.WORKLOADS["window_8k"]
    q, k, v = si.linear_inputs(wl)
    qw, kw = si.window_inputs(wl)
    qd, kd, vd, qwd, kwd = dev(q, k, v, qw, kw)
    y, _, _ = based.based_prefill(qd, kd, vd, chunk=wl.chunk, eps=wl.eps)
    based.swa_forward(qwd, kwd, vd, window=wl.window, scale=wl.swa_scale, add=y, y=y)
    torch.cuda.synchronize()
    want = oracle.la_recurrent(q, k, v, eps=wl.eps)[0] + oracle.swa(qw, kw, v, wl.window, wl.swa_scale)
    report("window_8k layer (all heads)", ratio(y, want), wl.tol)


@pytest.mark.timeout(900)
def test_workload_decode_1p3b():
    """The 1.3B decode workload: a 1024-token prefill (B=128, H=16, d_v=128)
    then 1024 next-token steps.  Every output of the prefill and of every
    step, for all 2048 heads, and the final state are compared with the
    oracle's recurrent form over the whole sequence (prefix followed by the
    step tokens: a step continues the sequence, the relation pin P6 checks
    for the oracle's own step routine), in blocks of 128 heads."""
    based = based_mod()
    wl = si.WORKLOADS["decode_1p3b"]
    q, k, v = si.linear_inputs(wl)
    y_pre, S, z = based.based_prefill(*dev(q, k, v), chunk=wl.chunk, eps=wl.eps)
    T = wl.decode_steps
    steps = [si.decode_inputs(wl, t) for t in range(T)]
    y_dec = torch.empty((T, wl.B, wl.H, wl.dv), dtype=torch.float32, device=DEV)
    for t in range(T):
        based.based_decode_step(*dev(*steps[t]), S, z, eps=wl.eps, y=y_dec[t])
    torch.cuda.synchronize()
    BH = wl.B * wl.H
    qa = torch.cat([q, torch.stack([s_[0] for s_ in steps], dim=2)], dim=2).reshape(BH, wl.L + T, wl.d)
    ka = torch.cat([k, torch.stack([s_[1] for s_ in steps], dim=2)], dim=2).reshape(BH, wl.L + T, wl.d)
    va = torch.cat([v, torch.stack([s_[2] for s_ in steps], dim=2)], dim=2).reshape(BH, wl.L + T, wl.dv)
    del steps
    y_pre = y_pre.reshape(BH, wl.L, wl.dv).cpu()
    y_dec = y_dec.permute(1, 2, 0, 3).reshape(BH, T, wl.dv).cpu()
    S = S.reshape(BH, -1, wl.dv).cpu()
    z = z.reshape(BH, -1).cpu()
    acc = {n: Streamed() for n in ("prefill y", "step y", "S", "z")}
    blk = 128
    for h0 in range(0, BH, blk):
        sl = slice(h0, h0 + blk)
        yo, So, zo = oracle.la_recurrent(qa[sl], ka[sl], va[sl], eps=wl.eps)
        acc["prefill y"].add(y_pre[sl], yo[:, :wl.L])
        acc["step y"].add(y_dec[sl], yo[:, wl.L:])
        acc["S"].add(S[sl], So)
        acc["z"].add(z[sl], zo)
    for n, a in acc.items():
        report(f"decode_1p3b {n} (all heads, {T} steps)", a.ratio(), wl.tol)
