"""fp64 CPU oracle for Taylor linear attention and sliding-window softmax.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package; the product path
(``linear_attention_sequence_taylor_amd``) never does.  The C source
(``oracle.c``) states each definition and the page section it follows; this
module only marshals arrays into ``liboracle.so`` (built by :func:`build`).

Every entry point takes torch tensors or numpy arrays of shape
``[B, H, L, d]`` (or ``[B, H, d]`` for a decode step), widens them exactly to
float64 and returns float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, IEEE fp)."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(src), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(ctypes.c_double)
        I, D = ctypes.c_int, ctypes.c_double
        lib.oracle_num_features.argtypes = [I]
        lib.oracle_num_features.restype = I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_taylor_features.argtypes = [P, I, P]
        lib.oracle_la_quadratic.argtypes = [P, P, P, I, I, I, I, D, P]
        lib.oracle_la_recurrent.argtypes = [P, P, P, I, I, I, I, D, P, P, P, P, P]
        lib.oracle_decode_step.argtypes = [P, P, P, I, I, I, D, P, P, P]
        lib.oracle_swa.argtypes = [P, P, P, I, I, I, I, I, D, P]
        lib.oracle_swa_cache_fill.argtypes = [P, P, I, I, I, I, I, P, P]
        lib.oracle_la_backward.argtypes = [P, P, P, P, I, I, I, I, D, P, P, P]
        lib.oracle_la_backward_recurrent.argtypes = [P, P, P, P, I, I, I, I, D, P, P, P]
        lib.oracle_swa_backward.argtypes = [P, P, P, P, I, I, I, I, I, D, P, P, P]
        lib.oracle_swa_decode_step.argtypes = [P, P, P, ctypes.POINTER(ctypes.c_longlong), I, I, I, I, D,
                                               P, P, P]
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact widening to a contiguous float64 numpy array (bf16/fp32 -> fp64)."""
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_features(d: int) -> int:
    return _load().oracle_num_features(d)


def num_threads() -> int:
    return _load().oracle_num_threads()


def taylor_features(x) -> np.ndarray:
    """phi(x) for one raw vector x[d]; see oracle.h for the feature order."""
    x = _f64(x).reshape(-1)
    out = np.empty(num_features(x.size), np.float64)
    _load().oracle_taylor_features(_ptr(x), x.size, _ptr(out))
    return out


def la_quadratic(q, k, v, eps: float = 1e-6) -> np.ndarray:
    """Closed-form O(L^2) causal Taylor linear attention; q,k [...,L,d], v [...,L,dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, L, d = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    y = np.empty(tuple(lead) + (L, dv), np.float64)
    _load().oracle_la_quadratic(_ptr(q), _ptr(k), _ptr(v), BH, L, d, dv, eps, _ptr(y))
    return y


def la_recurrent(q, k, v, eps: float = 1e-6, S0=None, z0=None, want_y: bool = True):
    """Token-by-token recurrent form with explicit features.

    Returns (y, S, z): y [...,L,dv] (None if want_y is False), final state
    S [...,F,dv] and z [...,F].  S0/z0 give an initial state (default zero).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, L, d = q.shape
    dv = v.shape[-1]
    F = num_features(d)
    BH = int(np.prod(lead)) if lead else 1
    S0, z0 = _f64(S0), _f64(z0)
    if S0 is not None:
        assert S0.shape == tuple(lead) + (F, dv), S0.shape
    if z0 is not None:
        assert z0.shape == tuple(lead) + (F,), z0.shape
    y = np.empty(tuple(lead) + (L, dv), np.float64) if want_y else None
    S = np.empty(tuple(lead) + (F, dv), np.float64)
    z = np.empty(tuple(lead) + (F,), np.float64)
    _load().oracle_la_recurrent(_ptr(q), _ptr(k), _ptr(v), BH, L, d, dv, eps,
                                _ptr(S0), _ptr(z0), _ptr(y), _ptr(S), _ptr(z))
    return y, S, z


def decode_step(q, k, v, S, z, eps: float = 1e-6):
    """One next-token step.  q,k [...,d], v [...,dv], S [...,F,dv], z [...,F].

    Returns (y, S_new, z_new); the inputs are not modified.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(S).copy()
    z = _f64(z).copy()
    *lead, d = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    y = np.empty(tuple(lead) + (dv,), np.float64)
    _load().oracle_decode_step(_ptr(q), _ptr(k), _ptr(v), BH, d, dv, eps, _ptr(S), _ptr(z), _ptr(y))
    return y, S, z


def swa(q, k, v, window: int = 64, scale: float | None = None) -> np.ndarray:
    """Brute-force causal sliding-window softmax attention (window keys incl. self)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, L, dqk = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    y = np.empty(tuple(lead) + (L, dv), np.float64)
    _load().oracle_swa(_ptr(q), _ptr(k), _ptr(v), BH, L, dqk, dv, int(window), float(scale), _ptr(y))
    return y


def swa_cache_fill(k, v, window: int = 64, k_cache=None, v_cache=None):
    """The window's key/value ring after a prefix k,v [...,L,*]: the token at
    position p in slot p mod window.  Slots the prefix does not reach keep
    the given caches' values (zeros by default).  Returns (k_cache, v_cache),
    [..., window, *] float64."""
    k, v = _f64(k), _f64(v)
    *lead, L, dqk = k.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    kc = np.zeros(tuple(lead) + (window, dqk)) if k_cache is None else _f64(k_cache).copy()
    vc = np.zeros(tuple(lead) + (window, dv)) if v_cache is None else _f64(v_cache).copy()
    _load().oracle_swa_cache_fill(_ptr(k), _ptr(v), BH, L, dqk, dv, int(window), _ptr(kc), _ptr(vc))
    return kc, vc


def swa_decode_step(q, k, v, k_cache, v_cache, pos, window: int = 64, scale: float | None = None):
    """One next-token step of the window.  q,k [B,H,dqk], v [B,H,dv], caches
    [B,H,window,*], pos [B] (position of each sequence's new token).
    Returns (y, k_cache_new, v_cache_new); the inputs are not modified."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    kc, vc = _f64(k_cache).copy(), _f64(v_cache).copy()
    B, H, dqk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    pos = np.ascontiguousarray(np.repeat(np.asarray(pos, dtype=np.int64).reshape(B), H), dtype=np.int64)
    assert (pos >= 0).all()
    y = np.empty((B, H, dv), np.float64)
    _load().oracle_swa_decode_step(_ptr(q), _ptr(k), _ptr(v),
                                   pos.ctypes.data_as(ctypes.POINTER(ctypes.c_longlong)),
                                   B * H, dqk, dv, int(window), float(scale), _ptr(kc), _ptr(vc), _ptr(y))
    return y, kc, vc


def la_backward(q, k, v, dy, eps: float = 1e-6):
    """Gradients (dq, dk, dv) of la_quadratic(q, k, v, eps) for the upstream
    gradient dy (shapes as the inputs and the output)."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    *lead, L, d = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dvo = np.empty_like(v)
    _load().oracle_la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dy), BH, L, d, dv, eps, _ptr(dq), _ptr(dk), _ptr(dvo))
    return dq, dk, dvo


def swa_backward(q, k, v, dy, window: int = 64, scale: float | None = None):
    """Gradients (dq, dk, dv) of swa(q, k, v, window, scale) for the upstream
    gradient dy (shapes as the inputs and the output)."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    *lead, L, dqk = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dvo = np.empty_like(v)
    _load().oracle_swa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dy), BH, L, dqk, dv, int(window), float(scale),
                                _ptr(dq), _ptr(dk), _ptr(dvo))
    return dq, dk, dvo


def la_backward_recurrent(q, k, v, dy, eps: float = 1e-6):
    """The gradients of la_backward by the recurrent (feature) form, O(L F dv)
    per head: a forward sweep with the state S, z and a backward sweep with
    the sums of phi(q_i) dy_i / D_i over later queries."""
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    *lead, L, d = q.shape
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dvo = np.empty_like(v)
    _load().oracle_la_backward_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(dy), BH, L, d, dv, eps, _ptr(dq),
                                         _ptr(dk), _ptr(dvo))
    return dq, dk, dvo
