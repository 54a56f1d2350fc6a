"""Random shapes for the oracle's own identities (hypothesis, derandomised so
that every run draws the same cases): the quadratic and recurrent forms
agree, prefill followed by next-token steps equals a longer prefill, the
two backward forms agree, and a window of at least L keys is plain causal
softmax attention."""
import numpy as np
import torch
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=25, deadline=None, derandomize=True)
shapes = st.tuples(st.integers(1, 2), st.integers(1, 2), st.integers(1, 70), st.sampled_from([8, 16, 24]),
                   st.integers(1, 9))


def _inputs(B, H, L, d, dv, seed, scale=0.7):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((B, H, L, d)), scale * rng.standard_normal((B, H, L, d)),
            rng.standard_normal((B, H, L, dv)))


@SETTINGS
@given(shapes, st.integers(0, 2 ** 31 - 1))
def test_quadratic_equals_recurrent(shape, seed):
    q, k, v = _inputs(*shape, seed)
    y_rec, _, _ = oracle.la_recurrent(q, k, v)
    np.testing.assert_allclose(oracle.la_quadratic(q, k, v), y_rec, rtol=1e-10, atol=1e-11)


@SETTINGS
@given(shapes, st.integers(1, 4), st.integers(0, 2 ** 31 - 1))
def test_decode_steps_continue_prefill(shape, T, seed):
    B, H, L, d, dv = shape
    q, k, v = _inputs(B, H, L + T, d, dv, seed)
    y_all, S_all, z_all = oracle.la_recurrent(q, k, v)
    _, S, z = oracle.la_recurrent(q[:, :, :L], k[:, :, :L], v[:, :, :L])
    for t in range(L, L + T):
        y, S, z = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S, z)
        np.testing.assert_allclose(y, y_all[:, :, t], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(S, S_all, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(z, z_all, rtol=1e-12, atol=1e-12)


@SETTINGS
@given(shapes, st.integers(0, 2 ** 31 - 1))
def test_backward_forms_agree(shape, seed):
    B, H, L, d, dv = shape
    q, k, v = _inputs(B, H, L, d, dv, seed, scale=0.5)
    dy = np.random.default_rng(seed + 1).standard_normal((B, H, L, dv))
    for a, b in zip(oracle.la_backward(q, k, v, dy), oracle.la_backward_recurrent(q, k, v, dy)):
        # gradients of early tokens come out of cancellations of terms of
        # order |dy||v|: compare against that scale
        np.testing.assert_allclose(b, a, rtol=1e-8, atol=1e-10 * max(1.0, float(np.abs(dy).max())))


@SETTINGS
@given(st.integers(1, 60), st.sampled_from([16, 64]), st.integers(1, 8), st.integers(0, 2 ** 31 - 1))
def test_wide_window_is_causal_softmax(L, dqk, dv, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((1, 2, L, n)) for n in (dqk, dqk, dv))
    scale = dqk ** -0.5
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = torch.ones(L, L, dtype=torch.bool).tril()
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale).numpy()
    for w in (L, L + 1, 10 * L):
        np.testing.assert_allclose(oracle.swa(q, k, v, w, scale), want, rtol=1e-10, atol=1e-12)
