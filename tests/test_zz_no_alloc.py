"""based_prefill_noalloc (the static-scratch variant of based_prefill, for
callers that cannot allocate) against based_prefill itself, through the C
ABI: two calls in a row that use the scratch, the second on a smaller
input, then a carried state; and the refusal of a call that needs more
scratch than the buffer holds."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2  # bf16 inputs: max error <= 2e-2 x RMS of the reference output


@pytest.fixture(scope="module")
def based():
    import linear_attention_sequence_taylor_amd as based  # fails loudly without the .so

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return based


def _ratio(got, want):
    got = got.detach().double().cpu()
    want = want.detach().double().cpu()
    return float((got - want).abs().max() / want.pow(2).mean().sqrt())


def _check(based, B, H, L, dv, seed, init=False):
    q, k, v = (t.to(DEV) for t in si.custom((B, H, L, 16), (B, H, L, dv), seed=seed, scale=0.5))
    kw = {}
    if init:
        qp, kp, vp = (t.to(DEV) for t in si.custom((B, H, 40, 16), (B, H, 40, dv), seed=seed + 5, scale=0.5))
        _, S0, z0 = based.based_prefill(qp, kp, vp)
        kw["initial_state"] = (S0, z0)
    nbytes = based.based_prefill_workspace_bytes(B, H, L, dv)
    assert nbytes > 0, "the shape must use the scratch"
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref = based.based_prefill(q, k, v, workspace=ws, **kw)
    # outputs pre-filled with NaN: every element must be written
    y, S, z = (torch.full_like(t, float("nan")) for t in ref)
    got = based.based_prefill_noalloc(q, k, v, y=y, S=S, z=z, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip("ySz", got, ref):
        r = _ratio(a, b)
        print(f"[noalloc] B={B} H={H} L={L} dv={dv} init={init} {name}: {r:.2e}", flush=True)
        assert r <= TOL, (name, r)
        assert torch.equal(a, b), f"{name}: the same launch plan must give the same bits"


def test_noalloc_matches_prefill(based):
    # long sequences with few heads: segment split through the scratch
    _check(based, 1, 4, 64 * 300 + 17, 64, seed=4000)
    _check(based, 1, 2, 1000, 128, seed=4010)  # second call, smaller input
    _check(based, 2, 3, 700, 64, seed=4020, init=True)  # carried state shared by column groups


def test_noalloc_refuses_oversized(based):
    # a carried state over many heads needs one scratch slot per head and
    # column group: more than the static buffer
    B, H, L, dv = 8, 256, 70, 128
    q, k, v = (t.to(DEV) for t in si.custom((B, H, L, 16), (B, H, L, dv), seed=4030, scale=0.5))
    S0 = torch.zeros(B, H, 273, dv, device=DEV)
    z0 = torch.ones(B, H, 273, device=DEV)
    with pytest.raises(based.BasedError, match="TOO_LARGE"):
        based.based_prefill_noalloc(q, k, v, initial_state=(S0, z0))
    # without the carried state the same shape needs no scratch and runs
    y, _, _ = based.based_prefill_noalloc(q, k, v)
    ref, _, _ = based.based_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
