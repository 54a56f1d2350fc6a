"""Pins for the fp64 oracle: checks against what the definitions and the
mathematics fix, never against the oracle itself.

Sources: "Simple linear attention language models balance the
recall-throughput tradeoff" (BASED) s2 (linear attention), s4 ("Taylor Linear
Attention", "Local Exact Attention"), App. B (prefill state handed to
next-token steps), App. D.4 ("State size": K-state denominator); "Gated Slot
Attention ..." App. A (recurrent matrix-valued state).

Which pin guards which part of the oracle:
  P1  feature map (order, pre-scale, 1/sqrt2): Taylor-of-exp limit and the
      closed-form kernel identity
  P2  la_quadratic vs la_recurrent (independent routines, one phi-free)
  P3  normaliser state invariants
  P4  special cases with closed forms (q=0, k=0, v const, linearity, columns)
  P5  window: library softmax attention with a band mask; w=1; w>=L
  P6  decode step and state handoff/resume
  P7  small-logit limit: linear attention -> softmax attention
  P8  window decode: ring cache filled from a prefix plus next-token steps
      equals the library's band-masked softmax attention at each position
  P9  gradients: torch autograd through a plain fp64 forward, and central
      finite differences of the oracle's own forward
  P11 window gradients: torch autograd through the library's band-masked
      softmax attention, central finite differences of the oracle's window,
      w = 1 (y = v), and the key-shift invariance of every row's softmax
  hand hand-worked rational cases in tests/golden/hand_cases.json
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _frac(s):
    return float(Fraction(s))


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("d", [4, 8, 16, 24, 32])
def test_p1_features_taylor_limit(oracle_mod, d):
    """phi(q).phi(k) must agree with exp(s), s = q.k/sqrt(d), up to the cubic
    term: (exp(s) - phi.phi) / s^3 -> 1/6 as s -> 0.  A wrong pre-scale, a
    missing 1/sqrt2, a dropped linear or constant term, or a transposed
    quadratic block changes the limit."""
    rng = _rng(d)
    for _ in range(5):
        u = rng.standard_normal(d)
        w = rng.standard_normal(d)
        for t in (1e-1, 3e-2, 1e-2):
            q, k = t * u, w
            s = float(q @ k) / math.sqrt(d)
            got = float(oracle_mod.taylor_features(q) @ oracle_mod.taylor_features(k))
            ratio = (math.exp(s) - got) / s**3
            assert abs(ratio - 1.0 / 6.0) < 0.2 * abs(s) + 1e-6, (d, t, ratio)


def test_p1_kernel_identity_random(oracle_mod):
    """phi(q).phi(k) = 1 + s + s^2/2 for large random q, k (exact identity)."""
    rng = _rng(1)
    for _ in range(50):
        q, k = 3 * rng.standard_normal(16), 3 * rng.standard_normal(16)
        s = float(q @ k) / 4.0
        got = float(oracle_mod.taylor_features(q) @ oracle_mod.taylor_features(k))
        assert abs(got - (1 + s + 0.5 * s * s)) <= 1e-13 * (1 + s * s)


def test_p1_feature_count(oracle_mod):
    assert oracle_mod.num_features(16) == 273
    assert oracle_mod.taylor_features(np.zeros(16)).shape == (273,)
    phi0 = oracle_mod.taylor_features(np.zeros(16))
    assert phi0[0] == 1.0 and not phi0[1:].any()


# ---------------------------------------------------------------- P2
@pytest.mark.parametrize("d", [8, 24, 32])
def test_p2_quadratic_equals_recurrent_feature_dims(oracle_mod, d):
    """The ablation feature sizes (BASED App. D.4): the phi-free closed form
    and the explicit (1 + d + d^2)-row recurrence agree for every d."""
    rng = _rng(100 + d)
    L = 45
    q = rng.standard_normal((1, 2, L, d))
    k = rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, 16))
    yq = oracle_mod.la_quadratic(q, k, v)
    yr, S, z = oracle_mod.la_recurrent(q, k, v)
    np.testing.assert_allclose(yq, yr, rtol=1e-11, atol=1e-12)
    assert S.shape[-2] == 1 + d + d * d and z[..., 0].tolist() == [[float(L)] * 2]


@pytest.mark.parametrize("L,dv", [(1, 64), (37, 64), (64, 128), (65, 64), (200, 128)])
def test_p2_quadratic_equals_recurrent(oracle_mod, L, dv):
    rng = _rng(L * 7 + dv)
    q = rng.standard_normal((2, 3, L, 16))
    k = rng.standard_normal((2, 3, L, 16))
    v = rng.standard_normal((2, 3, L, dv))
    yq = oracle_mod.la_quadratic(q, k, v)
    yr, _, _ = oracle_mod.la_recurrent(q, k, v)
    assert np.abs(yq - yr).max() <= 1e-12 * np.abs(yq).max()


def test_p2_tiny_workload_full(oracle_mod):
    from synthetic_inputs import WORKLOADS, linear_inputs

    wl = WORKLOADS["tiny_f32"]
    q, k, v = linear_inputs(wl)
    yq = oracle_mod.la_quadratic(q, k, v)
    yr, _, _ = oracle_mod.la_recurrent(q, k, v)
    assert np.abs(yq - yr).max() <= 1e-12 * np.abs(yq).max()


# ---------------------------------------------------------------- P3
def test_p3_normaliser_state(oracle_mod):
    rng = _rng(3)
    L = 50
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v = rng.standard_normal((1, 1, L, 8))
    _, S, z = oracle_mod.la_recurrent(q, k, v)
    z = z[0, 0]
    assert z[0] == L  # one unit per token, exactly
    np.testing.assert_allclose(z[1:17], k[0, 0].sum(0) * 16 ** -0.25, rtol=1e-13, atol=1e-13)
    Z = z[17:].reshape(16, 16)
    np.testing.assert_allclose(Z, Z.T, rtol=0, atol=1e-13)  # symmetric quadratic block
    assert np.all(np.diag(Z) >= 0)
    # S row 0 accumulates the raw values (constant feature)
    np.testing.assert_allclose(S[0, 0, 0], v[0, 0].sum(0), rtol=1e-13, atol=1e-12)


def test_p3_weights_at_least_half(oracle_mod):
    """1 + s + s^2/2 >= 1/2 for every s, so with v = e_c (one-hot column) the
    per-token weight sums are bounded: y_i[c] in [0, 1]."""
    rng = _rng(4)
    L = 40
    q = 2 * rng.standard_normal((1, 1, L, 16))
    k = 2 * rng.standard_normal((1, 1, L, 16))
    v = np.zeros((1, 1, L, 1))
    v[..., :] = 1.0
    y = oracle_mod.la_quadratic(q, k, v)
    assert np.all(y > 0.99) and np.all(y <= 1.0)


# ---------------------------------------------------------------- P4
def test_p4_zero_query_is_running_mean(oracle_mod):
    rng = _rng(5)
    L, dv, eps = 70, 16, 1e-6
    q = np.zeros((1, 2, L, 16))
    k = rng.standard_normal((1, 2, L, 16))
    v = rng.standard_normal((1, 2, L, dv))
    want = np.cumsum(v, axis=2) / (np.arange(1, L + 1)[:, None] + eps)
    for fn in (oracle_mod.la_quadratic, lambda *a: oracle_mod.la_recurrent(*a)[0]):
        np.testing.assert_allclose(fn(q, k, v), want, rtol=1e-12, atol=1e-14)
    # zero keys give the same weights (s = 0)
    np.testing.assert_allclose(oracle_mod.la_quadratic(k, q, v), want, rtol=1e-12, atol=1e-14)


def test_p4_constant_values(oracle_mod):
    rng = _rng(6)
    L = 90
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v = np.full((1, 1, L, 4), 2.5)
    y = oracle_mod.la_quadratic(q, k, v, eps=0.0)
    np.testing.assert_allclose(y, 2.5, rtol=1e-14)
    ys = oracle_mod.swa(q, k, v, window=64)
    np.testing.assert_allclose(ys, 2.5, rtol=1e-14)


def test_p4_linearity_and_columns(oracle_mod):
    rng = _rng(7)
    L = 60
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v1 = rng.standard_normal((1, 1, L, 8))
    v2 = rng.standard_normal((1, 1, L, 8))
    f = oracle_mod.la_quadratic
    np.testing.assert_allclose(f(q, k, 2 * v1 - 3 * v2), 2 * f(q, k, v1) - 3 * f(q, k, v2),
                               rtol=1e-12, atol=1e-12)
    perm = rng.permutation(8)
    np.testing.assert_allclose(f(q, k, v1[..., perm]), f(q, k, v1)[..., perm], rtol=1e-14, atol=0)
    fr = lambda *a: oracle_mod.la_recurrent(*a)[0]
    np.testing.assert_allclose(fr(q, k, v1[..., perm]), fr(q, k, v1)[..., perm], rtol=1e-14, atol=0)
    fs = lambda a, b, c: oracle_mod.swa(a, b, c, window=7)
    np.testing.assert_allclose(fs(q, k, 2 * v1 - 3 * v2), 2 * fs(q, k, v1) - 3 * fs(q, k, v2),
                               rtol=1e-12, atol=1e-12)


def test_p4_causality(oracle_mod):
    """Changing token t never changes outputs before t."""
    rng = _rng(8)
    L, t = 50, 31
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v = rng.standard_normal((1, 1, L, 8))
    y0 = oracle_mod.la_recurrent(q, k, v)[0]
    s0 = oracle_mod.swa(q, k, v, window=9)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[..., t, :] += 1
    k2[..., t, :] -= 2
    v2[..., t, :] *= 3
    y1 = oracle_mod.la_recurrent(q2, k2, v2)[0]
    s1 = oracle_mod.swa(q2, k2, v2, window=9)
    assert np.array_equal(y0[..., :t, :], y1[..., :t, :])
    assert np.array_equal(s0[..., :t, :], s1[..., :t, :])
    assert not np.allclose(y0[..., t:, :], y1[..., t:, :])


# ---------------------------------------------------------------- P5
def _sdpa_band(q, k, v, window, scale):
    """torch's softmax attention with an explicit causal band mask (fp64 CPU)."""
    L = q.shape[-2]
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    allowed = (j <= i) & (j > i - window)
    tq, tk, tv = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)
    return out.numpy()


@pytest.mark.parametrize("window,dqk", [(1, 16), (5, 16), (64, 64), (64, 16), (300, 64)])
def test_p5_window_matches_library_softmax(oracle_mod, window, dqk):
    rng = _rng(window + dqk)
    L = 150
    q = 2 * rng.standard_normal((2, 2, L, dqk))
    k = 2 * rng.standard_normal((2, 2, L, dqk))
    v = rng.standard_normal((2, 2, L, 32))
    scale = 1 / math.sqrt(dqk)
    got = oracle_mod.swa(q, k, v, window=window, scale=scale)
    np.testing.assert_allclose(got, _sdpa_band(q, k, v, window, scale), rtol=1e-11, atol=1e-12)


def test_p5_window_special_cases(oracle_mod):
    rng = _rng(9)
    L = 80
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v = rng.standard_normal((1, 1, L, 8))
    assert np.array_equal(oracle_mod.swa(q, k, v, window=1), v)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    full = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=0.25)
    np.testing.assert_allclose(oracle_mod.swa(q, k, v, window=L, scale=0.25), full.numpy(),
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(oracle_mod.swa(q, k, v, window=10 * L, scale=0.25), full.numpy(),
                               rtol=1e-11, atol=1e-12)
    # zero logits: plain mean over the window
    w = 6
    ys = oracle_mod.swa(np.zeros_like(q), k, v, window=w)
    for i in range(L):
        j0 = max(0, i - w + 1)
        np.testing.assert_allclose(ys[0, 0, i], v[0, 0, j0:i + 1].mean(0), rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- P6
def test_p6_decode_continues_prefill(oracle_mod):
    rng = _rng(10)
    L1, T = 45, 12
    q = rng.standard_normal((2, 2, L1 + T, 16))
    k = rng.standard_normal((2, 2, L1 + T, 16))
    v = rng.standard_normal((2, 2, L1 + T, 32))
    full = oracle_mod.la_quadratic(q, k, v)
    _, S, z = oracle_mod.la_recurrent(q[..., :L1, :], k[..., :L1, :], v[..., :L1, :])
    for t in range(L1, L1 + T):
        y, S, z = oracle_mod.decode_step(q[..., t, :], k[..., t, :], v[..., t, :], S, z)
        np.testing.assert_allclose(y, full[..., t, :], rtol=1e-11, atol=1e-13)


def test_p6_resume_from_state(oracle_mod):
    rng = _rng(11)
    L, cut = 77, 33
    q = rng.standard_normal((1, 3, L, 16))
    k = rng.standard_normal((1, 3, L, 16))
    v = rng.standard_normal((1, 3, L, 16))
    y_full, S_full, z_full = oracle_mod.la_recurrent(q, k, v)
    y_a, S_a, z_a = oracle_mod.la_recurrent(q[..., :cut, :], k[..., :cut, :], v[..., :cut, :])
    y_b, S_b, z_b = oracle_mod.la_recurrent(q[..., cut:, :], k[..., cut:, :], v[..., cut:, :], S0=S_a, z0=z_a)
    np.testing.assert_allclose(np.concatenate([y_a, y_b], axis=2), y_full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S_b, S_full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z_b, z_full, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- P8
@pytest.mark.parametrize("window,L", [(1, 5), (7, 0), (7, 3), (7, 30), (64, 10), (64, 64), (64, 150)])
def test_p8_window_decode_continues_window(oracle_mod, window, L):
    """The w-sized cache of the window [BASED s4 "Local Exact Attention"]:
    fill it from a prefix, then take next-token steps; every step equals
    torch's band-masked softmax attention over the whole sequence at that
    position.  The two sequences of the batch sit at different positions,
    and the caches start as NaN, so a slot read before it holds one of the
    last `window` tokens poisons the result."""
    rng = _rng(40 + window + L)
    B, H, dqk, dv, lag = 2, 2, 16, 8, 5
    T = 2 * window + 3
    n = L + lag + T
    q = 2 * rng.standard_normal((B, H, n, dqk))
    k = 2 * rng.standard_normal((B, H, n, dqk))
    v = rng.standard_normal((B, H, n, dv))
    scale = 1 / math.sqrt(dqk)
    full = _sdpa_band(q, k, v, window, scale)
    starts = [L, L + lag]
    kc = np.full((B, H, window, dqk), np.nan)
    vc = np.full((B, H, window, dv), np.nan)
    for b, L0 in enumerate(starts):
        kc[b], vc[b] = oracle_mod.swa_cache_fill(k[b:b + 1, :, :L0], v[b:b + 1, :, :L0], window,
                                                 kc[b:b + 1], vc[b:b + 1])
    for t in range(T):
        pos = np.array([L0 + t for L0 in starts])
        pick = lambda x: np.stack([x[b, :, pos[b]] for b in range(B)])
        y, kc, vc = oracle_mod.swa_decode_step(pick(q), pick(k), pick(v), kc, vc, pos, window, scale)
        np.testing.assert_allclose(y, pick(full), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- P9
def _torch_forward(q, k, v, eps):
    """The causal Taylor linear attention forward written with torch ops
    (fp64), for autograd to differentiate."""
    d = q.shape[-1]
    s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    a = (1 + s + 0.5 * s * s) * torch.tril(torch.ones(q.shape[-2], q.shape[-2], dtype=q.dtype))
    return (a @ v) / (a.sum(-1, keepdim=True) + eps)


@pytest.mark.parametrize("d,L,dv", [(16, 37, 8), (8, 20, 16), (16, 1, 4)])
def test_p9_backward_matches_autograd(oracle_mod, d, L, dv):
    rng = _rng(60 + d + L)
    q = rng.standard_normal((2, 2, L, d))
    k = rng.standard_normal((2, 2, L, d))
    v = rng.standard_normal((2, 2, L, dv))
    dy = rng.standard_normal((2, 2, L, dv))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    (_torch_forward(tq, tk, tv, 1e-6) * torch.from_numpy(dy)).sum().backward()
    dq, dk, dv_ = oracle_mod.la_backward(q, k, v, dy)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv_, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-11)


def test_p9_backward_finite_differences(oracle_mod):
    """Central differences of sum(y * dy), y from the oracle's closed-form
    forward, at random coordinates of q, k and v."""
    rng = _rng(70)
    L, d, dv = 23, 16, 6
    q = rng.standard_normal((1, 1, L, d))
    k = rng.standard_normal((1, 1, L, d))
    v = rng.standard_normal((1, 1, L, dv))
    dy = rng.standard_normal((1, 1, L, dv))
    grads = dict(zip("qkv", oracle_mod.la_backward(q, k, v, dy)))
    loss = lambda a, b, c: float((oracle_mod.la_quadratic(a, b, c) * dy).sum())
    h = 1e-5
    for name, x in (("q", q), ("k", k), ("v", v)):
        for _ in range(8):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(**{"a": args_p["q"], "b": args_p["k"], "c": args_p["v"]})
                  - loss(**{"a": args_m["q"], "b": args_m["k"], "c": args_m["v"]})) / (2 * h)
            assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


# ---------------------------------------------------------------- P10
@pytest.mark.parametrize("d,L,dv", [(16, 37, 8), (8, 20, 16), (16, 2, 4), (24, 9, 5)])
def test_p10_recurrent_backward_matches_autograd(oracle_mod, d, L, dv):
    """The recurrent-form backward (forward sweep for dq, reverse sweep for dk
    and dv) against autograd through the closed-form forward."""
    rng = _rng(80 + d + L)
    q = rng.standard_normal((2, 2, L, d))
    k = rng.standard_normal((2, 2, L, d))
    v = rng.standard_normal((2, 2, L, dv))
    dy = rng.standard_normal((2, 2, L, dv))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    (_torch_forward(tq, tk, tv, 1e-6) * torch.from_numpy(dy)).sum().backward()
    got = oracle_mod.la_backward_recurrent(q, k, v, dy)
    for g, want in zip(got, (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(g, want.numpy(), rtol=1e-9, atol=1e-10)


def test_p10_recurrent_backward_equals_closed_form(oracle_mod):
    """At a length spanning several 64-token chunks with a ragged tail, the
    two backward forms agree to rounding."""
    rng = _rng(90)
    L, d, dv = 150, 16, 64
    q = 0.5 * rng.standard_normal((1, 2, L, d))
    k = 0.5 * rng.standard_normal((1, 2, L, d))
    v = rng.standard_normal((1, 2, L, dv))
    dy = rng.standard_normal((1, 2, L, dv))
    for a, b in zip(oracle_mod.la_backward(q, k, v, dy), oracle_mod.la_backward_recurrent(q, k, v, dy)):
        np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-11 * np.abs(a).max())


# ---------------------------------------------------------------- P7
def test_p7_small_logits_approach_softmax(oracle_mod):
    """With q scaled by t -> 0 the Taylor weights approach exp(s); the gap to
    causal softmax attention (scale 1/sqrt(d')) shrinks like t^3."""
    rng = _rng(12)
    L = 40
    q = rng.standard_normal((1, 1, L, 16))
    k = rng.standard_normal((1, 1, L, 16))
    v = rng.standard_normal((1, 1, L, 8))
    errs = []
    for t in (0.4, 0.2, 0.1):
        y = oracle_mod.la_quadratic(t * q, k, v, eps=0.0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(t * q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True, scale=0.25)
        errs.append(np.abs(y - ref.numpy()).max())
    assert errs[1] < errs[0] / 5 and errs[2] < errs[1] / 5, errs


# ---------------------------------------------------------------- hand cases
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_hand_taylor_cases(oracle_mod):
    for case in _golden()["taylor"]:
        L, d = case["L"], case["d"]
        q = np.zeros((1, 1, L, d))
        k = np.zeros((1, 1, L, d))
        for t, a, val in case["q_nonzero"]:
            q[0, 0, t, a] = val
        for t, a, val in case["k_nonzero"]:
            k[0, 0, t, a] = val
        v = np.array(case["v"], np.float64)[None, None]
        want = np.array([[_frac(x) for x in row] for row in case["y"]])
        np.testing.assert_allclose(oracle_mod.la_quadratic(q, k, v, eps=case["eps"])[0, 0], want, rtol=1e-14)
        y, S, z = oracle_mod.la_recurrent(q, k, v, eps=case["eps"])
        np.testing.assert_allclose(y[0, 0], want, rtol=1e-13, atol=1e-15)
        for idx, val in case["z_checks"].items():
            num = val.split()[0]
            expect = _frac(num) / (math.sqrt(2) if "/sqrt2" in val else 1.0)
            assert abs(z[0, 0, int(idx)] - expect) < 1e-13


def test_hand_window_cases(oracle_mod):
    for case in _golden()["window"]:
        L = case["L"]
        q = np.zeros((1, 1, L, case["dqk"]))
        k = np.zeros((1, 1, L, case["dqk"]))
        q[..., 0] = 1.0
        k[0, 0, :, 0] = np.arange(L) * math.log(2.0)
        v = np.array(case["v"], np.float64)[None, None]
        for sub in case["cases"]:
            want = np.array([_frac(x) for x in sub["y"]])
            got = oracle_mod.swa(q, k, v, window=sub["window"], scale=case["scale"])[0, 0, :, 0]
            np.testing.assert_allclose(got, want, rtol=1e-14)


# ---------------------------------------------------------------- P11
def _sdpa_band_torch(tq, tk, tv, window, scale):
    L = tq.shape[-2]
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    allowed = (j <= i) & (j > i - window)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allowed, scale=scale)


@pytest.mark.parametrize("window,dqk,L", [(64, 64, 150), (5, 16, 40), (1, 8, 12), (300, 16, 70)])
def test_p11_window_backward_matches_autograd(oracle_mod, window, dqk, L):
    """The library's softmax attention (band mask, fp64) differentiated by
    autograd: an implementation of the forward that shares nothing with the
    oracle's loops."""
    rng = _rng(90 + window + dqk)
    q = 2 * rng.standard_normal((2, 2, L, dqk))
    k = 2 * rng.standard_normal((2, 2, L, dqk))
    v = rng.standard_normal((2, 2, L, 7))
    dy = rng.standard_normal((2, 2, L, 7))
    scale = 1 / math.sqrt(dqk)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    (_sdpa_band_torch(tq, tk, tv, window, scale) * torch.from_numpy(dy)).sum().backward()
    got = oracle_mod.swa_backward(q, k, v, dy, window, scale)
    for g, want in zip(got, (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(g, want.numpy(), rtol=1e-9, atol=1e-11)


def test_p11_window_backward_finite_differences(oracle_mod):
    """Central differences of sum(y * dy), y from the oracle's own window
    forward, at random coordinates of q, k and v."""
    rng = _rng(91)
    L, dqk, dv, window = 29, 8, 5, 6
    q = rng.standard_normal((1, 1, L, dqk))
    k = rng.standard_normal((1, 1, L, dqk))
    v = rng.standard_normal((1, 1, L, dv))
    dy = rng.standard_normal((1, 1, L, dv))
    grads = dict(zip("qkv", oracle_mod.swa_backward(q, k, v, dy, window, 0.4)))
    h = 1e-5
    for name, x in (("q", q), ("k", k), ("v", v)):
        for _ in range(10):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            args_p, args_m = dict(q=q, k=k, v=v), dict(q=q, k=k, v=v)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[name], args_m[name] = xp, xm
            fd = (float((oracle_mod.swa(**args_p, window=window, scale=0.4) * dy).sum())
                  - float((oracle_mod.swa(**args_m, window=window, scale=0.4) * dy).sum())) / (2 * h)
            assert abs(fd - grads[name][idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grads[name][idx])


def test_p11_window_backward_special_cases(oracle_mod):
    """w = 1: every query sees only its own key, y = v, so dq = dk = 0 and
    dv = dy exactly.  Any window: shifting every key by the same vector c
    moves each row's logits by one constant (q_i . c), which the softmax
    ignores, so the key gradients sum to zero over the sequence."""
    rng = _rng(92)
    q, k = rng.standard_normal((2, 1, 3, 33, 16))
    v, dy = rng.standard_normal((2, 1, 3, 33, 10))
    dq, dk, dv = oracle_mod.swa_backward(q, k, v, dy, 1, 0.25)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_array_equal(dv, dy)
    for window in (2, 7, 33, 100):
        dq, dk, dv = oracle_mod.swa_backward(q, k, v, dy, window, 0.25)
        np.testing.assert_allclose(dk.sum(axis=-2), 0.0, atol=1e-12 * max(1.0, np.abs(dk).max()) * 33)
        assert np.abs(dk).max() > 1e-3
