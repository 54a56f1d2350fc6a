"""Taylor linear attention (BASED) on MI355X: Python binding of libbased.so.

Thin marshalling over the C ABI in include/based.h: these functions check
device, dtype, shape and contiguity, allocate outputs with torch (device
memory only), pass raw pointers and the current HIP stream, and turn a
status code into an exception.  Every step of the computation runs in the
HIP kernels of libbased.so; nothing here computes.

    based_prefill(q, k, v)            -> (y, S, z)     prompt processing
    based_decode_step(q, k, v, S, z)  -> y             next-token step (S, z in place)
    swa_forward(q, k, v, window=64)   -> y             sliding-window softmax
    swa_cache_fill(k, v, window=64)   -> (kc, vc)      window key/value ring from a prefix
    swa_decode_step(q, k, v, kc, vc, pos) -> y         window next-token step (kc, vc in place)
    based_prefill_backward(q, k, v, dy) -> (dq, dk, dv) gradients of based_prefill's output
"""
from __future__ import annotations

import torch

from . import _lib

__all__ = ["based_prefill", "based_prefill_noalloc", "based_decode_step", "swa_forward", "swa_cache_fill", "swa_decode_step",
           "based_hybrid_prefill", "based_hybrid_prefill_workspace_bytes",
           "based_prefill_backward", "based_prefill_backward_workspace_bytes",
           "based_num_features", "based_prefill_workspace_bytes", "BasedError", "library_path"]

BasedError = _lib.BasedError
library_path = _lib.LIB_PATH
D_FEAT = 16

_DTYPES = {torch.float32: _lib.BASED_F32, torch.bfloat16: _lib.BASED_BF16}


def _stream_ptr(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name, t, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def _check_like(name, t, shape, dtype, device):
    """A caller-supplied tensor: contiguous, of the given dtype, exact shape
    and device (the kernels write or read all of it)."""
    _check_tensor(name, t, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")


def _workspace(ws, device):
    """(pointer, bytes) of a caller's workspace: a contiguous device tensor."""
    if ws is None:
        return None, 0
    _check_tensor("workspace", ws)
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _initial_state(initial_state, S, z):
    S0, z0 = initial_state
    if tuple(S0.shape) != tuple(S.shape) or tuple(z0.shape) != tuple(z.shape):
        raise ValueError(f"initial_state must have shapes {tuple(S.shape)} and {tuple(z.shape)}, "
                         f"got {tuple(S0.shape)} and {tuple(z0.shape)}")
    if S0.data_ptr() != S.data_ptr():
        S.copy_(S0)
    if z0.data_ptr() != z.data_ptr():
        z.copy_(z0)


def based_num_features(d_feat: int = D_FEAT) -> int:
    return _lib.lib().based_num_features(d_feat)


def based_prefill_workspace_bytes(B: int, H: int, L: int, d_v: int, d_feat: int = D_FEAT) -> int:
    return _lib.lib().based_prefill_workspace_bytes(B, H, L, d_feat, d_v)


def based_prefill_backward_workspace_bytes(B: int, H: int, L: int, d_v: int, d_feat: int = D_FEAT) -> int:
    return _lib.lib().based_prefill_backward_workspace_bytes(B, H, L, d_feat, d_v)


def based_prefill(q, k, v, *, chunk: int = 64, eps: float = 1e-6, initial_state=None,
                  y=None, S=None, z=None, workspace=None):
    """Causal Taylor linear attention over [B,H,L,*] inputs.

    Returns (y, S, z): y [B,H,L,d_v] fp32 and the final state S [B,H,273,d_v],
    z [B,H,273] (fp32).  ``initial_state=(S0, z0)`` starts from a carried
    state (copied into S, z unless they are the same tensors).  ``workspace``
    (a uint8 device tensor) enables the segment split for long sequences;
    by default one is allocated when the shape can use it.
    """
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 4)
    _check_tensor("v", v, dt, 4)
    B, H, L, d = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, H, L):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    F = 1 + d + d * d  # based_num_features(d), without a library round trip per call
    dev = q.device
    _check_device(dev, k=k, v=v)
    if y is None:
        y = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev)
    if S is None:
        S = torch.empty((B, H, F, d_v), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((B, H, F), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, L, d_v), torch.float32, dev)
    _check_like("S", S, (B, H, F, d_v), torch.float32, dev)
    _check_like("z", z, (B, H, F), torch.float32, dev)
    use_init = 0
    if initial_state is not None:
        _initial_state(initial_state, S, z)
        use_init = 1
    if workspace is None and chunk == 64:
        nbytes = based_prefill_workspace_bytes(B, H, L, d_v, d)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    st = _lib.lib().based_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, L, d,
                                  d_v, chunk, eps, y.data_ptr(), S.data_ptr(), z.data_ptr(), use_init,
                                  ws_ptr, ws_bytes, _stream_ptr(dev))
    _lib.check("based_prefill", st)
    return y, S, z


def based_prefill_noalloc(q, k, v, *, chunk: int = 64, eps: float = 1e-6, initial_state=None, y=None, S=None,
                          z=None):
    """based_prefill without a workspace: the library's static per-GPU
    scratch buffer stands in for it, and the C call allocates nothing (pass
    y, S, z to keep this function from allocating them).  Calls overlapping
    in time on one GPU race on that buffer.  Raises BasedError
    (BASED_E_TOO_LARGE) when the call needs more scratch than the buffer
    holds."""
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 4)
    _check_tensor("v", v, dt, 4)
    B, H, L, d = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, H, L):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    F = 1 + d + d * d
    dev = q.device
    _check_device(dev, k=k, v=v)
    if y is None:
        y = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev)
    if S is None:
        S = torch.empty((B, H, F, d_v), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((B, H, F), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, L, d_v), torch.float32, dev)
    _check_like("S", S, (B, H, F, d_v), torch.float32, dev)
    _check_like("z", z, (B, H, F), torch.float32, dev)
    use_init = 0
    if initial_state is not None:
        _initial_state(initial_state, S, z)
        use_init = 1
    st = _lib.lib().based_prefill_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, L, d, d_v,
                                          chunk, eps, y.data_ptr(), S.data_ptr(), z.data_ptr(), use_init,
                                          _stream_ptr(dev))
    _lib.check("based_prefill_noalloc", st)
    return y, S, z


def based_hybrid_prefill_workspace_bytes(B: int, H: int, L: int, d_v: int, d_feat: int = D_FEAT) -> int:
    return _lib.lib().based_hybrid_prefill_workspace_bytes(B, H, L, d_feat, d_v)


_HYBRID_PATHS = {"auto": 0, "fused": 1, "two_pass": 2}


def based_hybrid_prefill(q, k, q_win, k_win, v, *, chunk: int = 64, eps: float = 1e-6, window: int = 64,
                         scale: float | None = None, path: str = "auto", initial_state=None, y=None, S=None, z=None,
                         workspace=None):
    """The hybrid layer: Taylor linear attention of (q, k, v) plus the
    causal sliding-window softmax of (q_win, k_win, v), each normalised on
    its own.  ``path``: "auto" (the fused kernel wherever one exists),
    "fused" (error where none exists) or "two_pass".
    Returns (y, S, z) as ``based_prefill`` (S, z: the linear branch's final
    state)."""
    if path not in _HYBRID_PATHS:
        raise ValueError(f"path must be one of {sorted(_HYBRID_PATHS)}")
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for name, t in (("k", k), ("q_win", q_win), ("k_win", k_win), ("v", v)):
        _check_tensor(name, t, dt, 4)
    B, H, L, d = q.shape
    d_qk = q_win.shape[-1]
    d_v = v.shape[-1]
    if (k.shape != q.shape or k_win.shape != q_win.shape or q_win.shape[:3] != (B, H, L)
            or v.shape[:3] != (B, H, L)):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} q_win{tuple(q_win.shape)} "
                         f"k_win{tuple(k_win.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = d_qk ** -0.5
    F = 1 + d + d * d
    dev = q.device
    _check_device(dev, k=k, q_win=q_win, k_win=k_win, v=v)
    if y is None:
        y = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev)
    if S is None:
        S = torch.empty((B, H, F, d_v), dtype=torch.float32, device=dev)
    if z is None:
        z = torch.empty((B, H, F), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, L, d_v), torch.float32, dev)
    _check_like("S", S, (B, H, F, d_v), torch.float32, dev)
    _check_like("z", z, (B, H, F), torch.float32, dev)
    use_init = 0
    if initial_state is not None:
        _initial_state(initial_state, S, z)
        use_init = 1
    if workspace is None and chunk == 64:
        nbytes = based_hybrid_prefill_workspace_bytes(B, H, L, d_v, d)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    st = _lib.lib().based_hybrid_prefill(q.data_ptr(), k.data_ptr(), q_win.data_ptr(), k_win.data_ptr(),
                                         v.data_ptr(), _DTYPES[dt], B, H, L, d, d_qk, d_v, chunk, eps, window,
                                         scale, _HYBRID_PATHS[path], y.data_ptr(), S.data_ptr(), z.data_ptr(),
                                         use_init, ws_ptr, ws_bytes, _stream_ptr(dev))
    _lib.check("based_hybrid_prefill", st)
    return y, S, z


def based_decode_step(q, k, v, S, z, *, eps: float = 1e-6, y=None):
    """One next-token step: q,k [B,H,16], v [B,H,d_v]; S [B,H,273,d_v] and
    z [B,H,273] (fp32) are updated in place.  Returns y [B,H,d_v] fp32."""
    _check_tensor("q", q, ndim=3)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 3)
    _check_tensor("v", v, dt, 3)
    _check_tensor("S", S, torch.float32, 4)
    _check_tensor("z", z, torch.float32, 3)
    B, H, d = q.shape
    d_v = v.shape[-1]
    F = 1 + d + d * d
    dev = q.device
    if k.shape != q.shape or v.shape[:2] != (B, H):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _check_device(dev, k=k, v=v)
    _check_like("S", S, (B, H, F, d_v), torch.float32, dev)
    _check_like("z", z, (B, H, F), torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, d_v), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, d_v), torch.float32, dev)
    st = _lib.lib().based_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, d,
                                      d_v, eps, S.data_ptr(), z.data_ptr(), y.data_ptr(),
                                      _stream_ptr(q.device))
    _lib.check("based_decode_step", st)
    return y


def swa_forward(q, k, v, *, window: int = 64, scale: float | None = None, add=None, y=None):
    """Causal sliding-window softmax attention (window keys including self),
    plus ``add`` (fp32, same shape as the output) if given.  ``add`` may be
    ``y`` itself for an in-place accumulate.  Returns y [B,H,L,d_v] fp32."""
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 4)
    _check_tensor("v", v, dt, 4)
    B, H, L, d_qk = q.shape
    d_v = v.shape[-1]
    dev = q.device
    if k.shape != q.shape or v.shape[:3] != (B, H, L):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _check_device(dev, k=k, v=v)
    if scale is None:
        scale = d_qk ** -0.5
    if y is None:
        y = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, L, d_v), torch.float32, dev)
    if add is not None:
        _check_like("add", add, (B, H, L, d_v), torch.float32, dev)
    st = _lib.lib().swa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, L, d_qk,
                                d_v, int(window), float(scale), None if add is None else add.data_ptr(),
                                y.data_ptr(), _stream_ptr(q.device))
    _lib.check("swa_forward", st)
    return y


def swa_cache_fill(k, v, *, window: int = 64, k_cache=None, v_cache=None):
    """The window's key/value ring after a prefix k [B,H,L,d_qk], v [B,H,L,d_v]:
    the token at position p in slot p mod window (the last min(L, window)
    tokens are written, other slots are left as they are).  Returns
    (k_cache, v_cache), [B,H,window,d] in the inputs' dtype."""
    _check_tensor("k", k, ndim=4)
    dt = k.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("v", v, dt, 4)
    B, H, L, d_qk = k.shape
    d_v = v.shape[-1]
    if v.shape[:3] != (B, H, L):
        raise ValueError(f"shape mismatch k{tuple(k.shape)} v{tuple(v.shape)}")
    _check_device(k.device, v=v, k_cache=k_cache, v_cache=v_cache)
    if k_cache is None:
        k_cache = torch.zeros((B, H, window, d_qk), dtype=dt, device=k.device)
    if v_cache is None:
        v_cache = torch.zeros((B, H, window, d_v), dtype=dt, device=k.device)
    _check_tensor("k_cache", k_cache, dt, 4)
    _check_tensor("v_cache", v_cache, dt, 4)
    if tuple(k_cache.shape) != (B, H, window, d_qk) or tuple(v_cache.shape) != (B, H, window, d_v):
        raise ValueError("cache shapes must be [B,H,window,d]")
    st = _lib.lib().swa_cache_fill(k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, L, d_qk, d_v, int(window),
                                   k_cache.data_ptr(), v_cache.data_ptr(), _stream_ptr(k.device))
    _lib.check("swa_cache_fill", st)
    return k_cache, v_cache


def swa_decode_step(q, k, v, k_cache, v_cache, pos, *, scale: float | None = None, add=None, y=None):
    """Next-token step of the window for the tokens at positions pos [B]
    (int64 device tensor, not modified): q,k [B,H,d_qk], v [B,H,d_v] enter
    their slot of the caches [B,H,window,*] (updated in place), and
    y [B,H,d_v] fp32 is the softmax attention over the last `window` tokens
    (+ ``add``, which may be ``y``).  window = k_cache.shape[2]."""
    _check_tensor("q", q, ndim=3)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 3)
    _check_tensor("v", v, dt, 3)
    _check_tensor("k_cache", k_cache, dt, 4)
    _check_tensor("v_cache", v_cache, dt, 4)
    _check_tensor("pos", pos, torch.int64, 1)
    B, H, d_qk = q.shape
    d_v = v.shape[-1]
    window = k_cache.shape[2]
    if k.shape != q.shape or v.shape[:2] != (B, H) or pos.shape[0] != B:
        raise ValueError("shape mismatch")
    if tuple(k_cache.shape) != (B, H, window, d_qk) or tuple(v_cache.shape) != (B, H, window, d_v):
        raise ValueError("cache shapes must be [B,H,window,d]")
    dev = q.device
    _check_device(dev, k=k, v=v, k_cache=k_cache, v_cache=v_cache, pos=pos)
    if scale is None:
        scale = d_qk ** -0.5
    if y is None:
        y = torch.empty((B, H, d_v), dtype=torch.float32, device=dev)
    _check_like("y", y, (B, H, d_v), torch.float32, dev)
    if add is not None:
        _check_like("add", add, (B, H, d_v), torch.float32, dev)
    st = _lib.lib().swa_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _DTYPES[dt], B, H, d_qk, d_v,
                                    int(window), float(scale), pos.data_ptr(), k_cache.data_ptr(),
                                    v_cache.data_ptr(), None if add is None else add.data_ptr(), y.data_ptr(),
                                    _stream_ptr(q.device))
    _lib.check("swa_decode_step", st)
    return y


_BACKWARD_FORMS = {"auto": 0, "direct": 1, "chunked": 2}


def based_prefill_backward(q, k, v, dy, *, eps: float = 1e-6, form: str = "auto", dq=None, dk=None, dv=None,
                           workspace=None):
    """Gradients (dq, dk, dv), fp32, of based_prefill's output y for the
    upstream gradient dy [B,H,L,d_v] (fp32), from a zero initial state.
    ``form``: "direct" (pair by pair, O(L^2)), "chunked" (linear in L through
    the carried state; bf16, d' = 16) or "auto" (chunked where it
    is supported and faster)."""
    if form not in _BACKWARD_FORMS:
        raise ValueError(f"form must be one of {sorted(_BACKWARD_FORMS)}")
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 4)
    _check_tensor("v", v, dt, 4)
    _check_tensor("dy", dy, torch.float32, 4)
    B, H, L, d = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, H, L) or dy.shape != v.shape:
        raise ValueError("shape mismatch")
    dev = q.device
    _check_device(dev, k=k, v=v, dy=dy)
    dq = torch.empty((B, H, L, d), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty((B, H, L, d), dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev) if dv is None else dv
    _check_like("dq", dq, (B, H, L, d), torch.float32, dev)
    _check_like("dk", dk, (B, H, L, d), torch.float32, dev)
    _check_like("dv", dv, (B, H, L, d_v), torch.float32, dev)
    if workspace is None:
        nbytes = based_prefill_backward_workspace_bytes(B, H, L, d_v, d)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    st = _lib.lib().based_prefill_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dy.data_ptr(), _DTYPES[dt], B,
                                           H, L, d, d_v, eps, _BACKWARD_FORMS[form], dq.data_ptr(), dk.data_ptr(),
                                           dv.data_ptr(),
                                           ws_ptr, ws_bytes, _stream_ptr(dev))
    _lib.check("based_prefill_backward", st)
    return dq, dk, dv


def swa_backward_workspace_bytes(B: int, H: int, L: int) -> int:
    return _lib.lib().based_swa_backward_workspace_bytes(B, H, L)


def swa_backward(q, k, v, dy, *, window: int = 64, scale: float | None = None, dq=None, dk=None, dv=None,
                 workspace=None):
    """Gradients (dq, dk, dv), fp32, of swa_forward's output for the upstream
    gradient dy [B,H,L,d_v] (fp32): bf16 q, k [B,H,L,64], v [B,H,L,d_v]
    with d_v 64 or 128, windows 1..64."""
    _check_tensor("q", q, ndim=4)
    dt = q.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    _check_tensor("k", k, dt, 4)
    _check_tensor("v", v, dt, 4)
    _check_tensor("dy", dy, torch.float32, 4)
    B, H, L, d_qk = q.shape
    d_v = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, H, L) or dy.shape != v.shape:
        raise ValueError("shape mismatch")
    dev = q.device
    _check_device(dev, k=k, v=v, dy=dy)
    if scale is None:
        scale = d_qk ** -0.5
    dq = torch.empty((B, H, L, d_qk), dtype=torch.float32, device=dev) if dq is None else dq
    dk = torch.empty((B, H, L, d_qk), dtype=torch.float32, device=dev) if dk is None else dk
    dv = torch.empty((B, H, L, d_v), dtype=torch.float32, device=dev) if dv is None else dv
    _check_like("dq", dq, (B, H, L, d_qk), torch.float32, dev)
    _check_like("dk", dk, (B, H, L, d_qk), torch.float32, dev)
    _check_like("dv", dv, (B, H, L, d_v), torch.float32, dev)
    if workspace is None:
        workspace = torch.empty(max(swa_backward_workspace_bytes(B, H, L), 16), dtype=torch.uint8, device=dev)
    ws_ptr, ws_bytes = _workspace(workspace, dev)
    st = _lib.lib().based_swa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), dy.data_ptr(), _DTYPES[dt], B, H, L,
                                       d_qk, d_v, int(window), float(scale), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(dev))
    _lib.check("based_swa_backward", st)
    return dq, dk, dv
