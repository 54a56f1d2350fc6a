"""Randomised small shapes, seeded: each case draws its shape, input type and
options from its own fixed generator, runs the library call on the GPU and
compares every element with the oracle at the bar of the input type (2e-2 of
the oracle output's RMS for bf16 inputs, 1e-4 for fp32).  Each case prints
what it drew before it runs, so a failure names its shape."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16, F32 = torch.bfloat16, torch.float32


@pytest.fixture(scope="module")
def based():
    oracle.build()
    import linear_attention_sequence_taylor_amd as based  # fails loudly without the .so

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return based


def _ratio(got, want):
    got = got.detach().cpu().double().numpy()
    want = np.asarray(want, np.float64)
    return float(np.abs(got - want).max()) / float(np.sqrt(np.mean(want ** 2)))


def _check(name, got, want, tol):
    r = _ratio(got, want)
    print(f"[property] {name}: {r:.3e} (bar {tol:.0e})", flush=True)
    assert r <= tol, f"{name}: {r:.3e} > {tol:.0e}"


def _dev(*ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("case", range(24))
def test_random_prefill(based, case):
    """based_prefill at a random (B, H, L, d', d_v, input type, chunk, input
    scale), with or without a carried initial state, against the oracle's
    recurrent form (y, S and z)."""
    rng = np.random.default_rng(7000 + case)
    B, H = (int(x) for x in rng.integers(1, 4, 2))
    L = int(rng.integers(1, 400))
    d = int(rng.choice([8, 16, 24, 32]))
    dv = int(rng.choice([64, 128]))
    dtype = BF16 if rng.random() < 0.6 else F32
    chunk = 64 if (dtype == BF16 and d == 16) else int(rng.choice([16, 32, 64]))
    scale = float(rng.uniform(0.3, 1.2))
    with_init = bool(rng.random() < 0.4)
    print(f"[property] prefill case {case}: B={B} H={H} L={L} d={d} dv={dv} {dtype} chunk={chunk} "
          f"scale={scale:.2f} init={with_init}", flush=True)
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=7100 + 3 * case, scale=scale, dtype=dtype)
    S0 = z0 = None
    init = None
    if with_init:  # a state from an independent random prefix, by the oracle
        pq, pk, pv = si.custom((B, H, 37, d), (B, H, 37, dv), seed=7200 + 3 * case, scale=scale, dtype=dtype)
        _, S0, z0 = oracle.la_recurrent(pq, pk, pv, want_y=False)
        init = (torch.from_numpy(S0).float().to(DEV), torch.from_numpy(z0).float().to(DEV))
    y, S, z = based.based_prefill(*_dev(q, k, v), chunk=chunk, initial_state=init)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    tol = 2e-2 if dtype == BF16 else 1e-4
    _check(f"prefill case {case} y", y, yo, tol)
    _check(f"prefill case {case} S", S, So, tol)
    _check(f"prefill case {case} z", z, zo, tol)


@pytest.mark.parametrize("case", range(6))
def test_random_long_prefill_fp32_path(based, case):
    """The fp32 matrix-core prefill on few heads and long sequences, where it
    splits each head into segments (random count and ragged last segment),
    with or without a carried initial state, against the oracle (y, S, z)."""
    rng = np.random.default_rng(7600 + case)
    B, H = (int(x) for x in rng.integers(1, 3, 2))
    L = int(rng.integers(1024, 3000))
    d = int(rng.choice([8, 24, 32]))
    dv = int(rng.choice([64, 128]))
    dtype = BF16 if rng.random() < 0.5 else F32
    if dtype == F32 and rng.random() < 0.3:
        d = 16
    with_init = bool(rng.random() < 0.5)
    print(f"[property] long fp32-path prefill case {case}: B={B} H={H} L={L} d={d} dv={dv} {dtype} "
          f"init={with_init}", flush=True)
    assert based.based_prefill_workspace_bytes(B, H, L, dv, d) > 0, "expected a segment split"
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=7700 + 3 * case, scale=0.5, dtype=dtype)
    S0 = z0 = init = None
    if with_init:
        pq, pk, pv = si.custom((B, H, 37, d), (B, H, 37, dv), seed=7800 + 3 * case, scale=0.5, dtype=dtype)
        _, S0, z0 = oracle.la_recurrent(pq, pk, pv, want_y=False)
        init = (torch.from_numpy(S0).float().to(DEV), torch.from_numpy(z0).float().to(DEV))
    y, S, z = based.based_prefill(*_dev(q, k, v), initial_state=init)
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v, S0=S0, z0=z0)
    tol = 2e-2 if dtype == BF16 else 1e-4
    _check(f"long fp32-path prefill case {case} y", y, yo, tol)
    _check(f"long fp32-path prefill case {case} S", S, So, tol)
    _check(f"long fp32-path prefill case {case} z", z, zo, tol)


@pytest.mark.parametrize("case", range(16))
def test_random_decode_continues_prefill(based, case):
    """A random prefix through based_prefill, then a random number of
    next-token steps, against the oracle's prefill over the whole sequence
    (outputs of the steps and the final state)."""
    rng = np.random.default_rng(7300 + case)
    B, H = (int(x) for x in rng.integers(1, 4, 2))
    L = int(rng.integers(1, 200))
    T = int(rng.integers(1, 6))
    d = int(rng.choice([8, 16, 24, 32]))
    dv = int(rng.choice([64, 128]))
    dtype = BF16 if rng.random() < 0.6 else F32
    print(f"[property] decode case {case}: B={B} H={H} L={L} steps={T} d={d} dv={dv} {dtype}", flush=True)
    q, k, v = si.custom((B, H, L + T, d), (B, H, L + T, dv), seed=7400 + 3 * case, scale=0.7, dtype=dtype)
    _, S, z = based.based_prefill(*_dev(q[:, :, :L], k[:, :, :L], v[:, :, :L]))
    ys = []
    for t in range(L, L + T):
        ys.append(based.based_decode_step(*_dev(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                                v[:, :, t].contiguous()), S, z))
    torch.cuda.synchronize()
    yo, So, zo = oracle.la_recurrent(q, k, v)
    tol = 2e-2 if dtype == BF16 else 1e-4
    _check(f"decode case {case} y", torch.stack(ys, 2), yo[:, :, L:], tol)
    _check(f"decode case {case} S", S, So, tol)
    _check(f"decode case {case} z", z, zo, tol)


@pytest.mark.parametrize("case", range(20))
def test_random_window(based, case):
    """swa_forward at a random (B, H, L, d_qk, d_v, window, scale, input
    type), with or without a fused add, against brute-force softmax."""
    rng = np.random.default_rng(7500 + case)
    B, H = (int(x) for x in rng.integers(1, 4, 2))
    L = int(rng.integers(1, 500))
    dqk = int(rng.choice([16, 64]))
    dv = int(rng.choice([64, 128]))
    window = int(rng.choice([1, 2, int(rng.integers(3, 64)), 64, int(rng.integers(65, 300)), 1 << 20]))
    dtype = BF16 if rng.random() < 0.6 else F32
    scale = float(rng.uniform(0.05, 0.4))
    with_add = bool(rng.random() < 0.5)
    print(f"[property] window case {case}: B={B} H={H} L={L} dqk={dqk} dv={dv} w={window} {dtype} "
          f"scale={scale:.3f} add={with_add}", flush=True)
    q, k, v = si.custom((B, H, L, dqk), (B, H, L, dv), seed=7600 + 3 * case, scale=1.0, dtype=dtype)
    add = si.randn((B, H, L, dv), 7700 + case, 1.0, F32) if with_add else None
    y = based.swa_forward(*_dev(q, k, v), window=window, scale=scale, add=None if add is None else add.to(DEV))
    torch.cuda.synchronize()
    want = oracle.swa(q, k, v, window, scale)
    if add is not None:
        want = want + add.double().numpy()
    _check(f"window case {case}", y, want, 2e-2 if dtype == BF16 else 1e-4)


@pytest.mark.parametrize("case", range(16))
def test_random_backward(based, case):
    """based_prefill_backward at a random shape and input type, in the form
    the case draws (the chunked form where it applies), against the oracle's
    chain rule."""
    rng = np.random.default_rng(7800 + case)
    B, H = (int(x) for x in rng.integers(1, 3, 2))
    L = int(rng.integers(1, 300))
    d = int(rng.choice([8, 16, 24, 32]))
    dv = int(rng.choice([64, 128]))
    dtype = BF16 if rng.random() < 0.6 else F32
    form = "direct"
    if rng.random() < 0.6:  # the chunked form's inputs
        d, dtype, form = 16, BF16, "chunked"
    if L == 1:
        L = 2  # at L = 1, dq and dk are rounding noise (tested on their own)
    print(f"[property] backward case {case}: B={B} H={H} L={L} d={d} dv={dv} {dtype} {form}", flush=True)
    q, k, v = si.custom((B, H, L, d), (B, H, L, dv), seed=7900 + 3 * case, scale=0.5, dtype=dtype)
    dy = si.randn((B, H, L, dv), 8000 + case, 1.0, F32)
    dq, dk, dv_ = based.based_prefill_backward(*_dev(q, k, v), dy.to(DEV), form=form)
    torch.cuda.synchronize()
    oq, ok, ov = oracle.la_backward(q, k, v, dy)
    tol = 2e-2 if dtype == BF16 else 1e-4
    _check(f"backward case {case} dq", dq, oq, tol)
    _check(f"backward case {case} dk", dk, ok, tol)
    _check(f"backward case {case} dv", dv_, ov, tol)
