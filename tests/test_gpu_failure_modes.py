"""Non-finite inputs and alternative launch plans.

* NaN or Inf in an input propagates to the outputs and state the input
  can reach and nowhere else: other heads stay bit-identical to a clean
  run, rows before the affected chunk (or window) are untouched, and no call
  hangs or faults.  The tensors are built on the CPU.
* The same heads run under different launch plans (32- or 64-column
  groups, with or without sequence segments and workspace) must each match
  the oracle: a race in the LDS pipeline of one plan would show as a
  mismatch in that plan only.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def based():
    oracle.build()
    import linear_attention_sequence_taylor_amd as based  # fails loudly without the .so

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return based


def _dev(*ts):
    return [t.to(DEV) for t in ts]


def _same(a, b):
    """Bitwise equality, NaN included."""
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("where,val", [("v", float("nan")), ("k", float("inf")), ("q", float("nan")),
                                       ("k", float("nan"))])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_nonfinite_input(based, where, val, dtype):
    B, H, L, p = 1, 3, 300, 150
    q, k, v = si.custom((B, H, L, 16), (B, H, L, 64), seed=3000, scale=0.5, dtype=dtype)
    clean = [t.clone() for t in based.based_prefill(*_dev(q, k, v))]
    bad = {"q": q.clone(), "k": k.clone(), "v": v.clone()}
    bad[where][0, 1, p, 0] = val
    y, S, z = based.based_prefill(*_dev(bad["q"], bad["k"], bad["v"]))
    torch.cuda.synchronize()
    for h in (0, 2):
        assert _same(y[0, h], clean[0][0, h]) and _same(S[0, h], clean[1][0, h]) and _same(z[0, h], clean[2][0, h])
    c0 = (p // 64) * 64  # first row of the affected chunk
    assert _same(y[0, 1, :c0], clean[0][0, 1, :c0])
    if where == "q":
        # a query reaches only its own output row
        assert not torch.isfinite(y[0, 1, p]).any()
        assert torch.isfinite(y[0, 1, p + 1:]).all()
        assert _same(S[0, 1], clean[1][0, 1]) and _same(z[0, 1], clean[2][0, 1])
    else:
        # every later row of the head has a non-finite element
        assert not torch.isfinite(y[0, 1, p:]).all(dim=-1).any(), "a row at or after the input stayed finite"
        assert not torch.isfinite(S[0, 1]).all()


@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_decode_nonfinite_input(based, where):
    B, H, d, dv = 2, 3, 16, 128
    q, k, v = si.custom((B, H, 40, d), (B, H, 40, dv), seed=3010, scale=1.0)
    _, S0, z0 = based.based_prefill(*_dev(q, k, v))
    qt, kt, vt = si.custom((B, H, d), (B, H, dv), seed=3011)
    Sc, zc = S0.clone(), z0.clone()
    yc = based.based_decode_step(*_dev(qt, kt, vt), Sc, zc)
    bad = {"q": qt.clone(), "k": kt.clone(), "v": vt.clone()}
    bad[where][1, 2, 3] = float("nan")
    S, z = S0.clone(), z0.clone()
    y = based.based_decode_step(*_dev(bad["q"], bad["k"], bad["v"]), S, z)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (0, 2), (1, 0), (1, 1)):
        assert _same(y[b, h], yc[b, h]) and _same(S[b, h], Sc[b, h]) and _same(z[b, h], zc[b, h])
    if where == "q":
        # the query enters every column of the readout, not the update
        assert torch.isnan(y[1, 2]).all()
        assert _same(S[1, 2], Sc[1, 2]) and _same(z[1, 2], zc[1, 2])
    elif where == "k":
        # features with k_3 are NaN: every state column and the normaliser
        assert torch.isnan(y[1, 2]).all()
        assert torch.isnan(S[1, 2]).any(dim=0).all() and torch.isnan(z[1, 2]).any()
    else:
        # v column 3 reaches state column 3 and output column 3 only
        keep = [c for c in range(128) if c != 3]
        assert torch.isnan(y[1, 2, 3]) and _same(y[1, 2, keep], yc[1, 2, keep])
        assert torch.isnan(S[1, 2, :, 3]).all() and _same(S[1, 2][:, keep], Sc[1, 2][:, keep])
        assert _same(z[1, 2], zc[1, 2])


@pytest.mark.parametrize("window", [64, 300])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_window_nonfinite_input(based, window, dtype):
    B, H, L, p = 1, 2, 700, 400
    q, k, v = si.custom((B, H, L, 64), (B, H, L, 64), seed=3020, scale=1.0, dtype=dtype)
    clean = based.swa_forward(*_dev(q, k, v), window=window).clone()
    vb = v.clone()
    vb[0, 1, p, 5] = float("nan")
    y = based.swa_forward(*_dev(q, k, vb), window=window)
    torch.cuda.synchronize()
    assert _same(y[0, 0], clean[0, 0])
    t0 = (p // 64) * 64  # first row of the affected tile
    assert _same(y[0, 1, :t0], clean[0, 1, :t0])
    # the rows whose window holds position p: column 5 is NaN
    assert torch.isnan(y[0, 1, p:min(L, p + window), 5]).all()
    end = ((p + window - 1) // 64 + 1) * 64  # past the last tile the NaN key reaches
    assert _same(y[0, 1, end:], clean[0, 1, end:])


def _ratio(got, want):
    got = got.detach().cpu().double().numpy()
    return float(np.abs(got - want).max() / np.sqrt(np.mean(want ** 2)))


def test_prefill_launch_plans_agree(based):
    """Heads of a 360M-shaped layer (L = 2048) run as a 128-head call (32-column
    groups, no segments), as a 2-head call (64-column groups with sequence
    segments through the workspace) and as a 2-head call with no workspace
    (64-column groups, whole sequence): each against the oracle."""
    wl = si.WORKLOADS["prefill_360m"]
    q, k, v = si.linear_inputs(wl)
    q, k, v = (t.reshape(1, wl.B * wl.H, wl.L, -1) for t in (q, k, v))
    y_all, S_all, _ = based.based_prefill(*_dev(q, k, v))
    pick = [5, 77]
    sub = [t[:, pick].contiguous() for t in (q, k, v)]
    y_seg, S_seg, _ = based.based_prefill(*_dev(*sub))
    y_one, S_one, _ = based.based_prefill(*_dev(*sub), workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    yo, So, _ = oracle.la_recurrent(*sub)
    for name, y, S in (("128 heads", y_all[:, pick], S_all[:, pick]), ("segments", y_seg, S_seg),
                       ("whole sequence", y_one, S_one)):
        ry, rS = _ratio(y, yo), _ratio(S, So)
        print(f"[plans] {name}: y {ry:.3e} S {rS:.3e}", flush=True)
        assert ry <= wl.tol and rS <= wl.tol, (name, ry, rS)
