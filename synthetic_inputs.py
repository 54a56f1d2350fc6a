"""Seeded synthetic inputs shaped like BASED-360M / 1.3B attention layers.

This module holds the workload shapes and the random-number recipe only; it
contains none of the method's arithmetic.  Both the HIP path and the fp64
oracle consume the same tensors from here.

Recipe (one torch CPU generator per tensor):
  * ``torch.Generator('cpu').manual_seed(seed)``; draw fp32 ``randn``; multiply
    by the workload's scale; for bf16 workloads round with ``.to(bfloat16)``
    (round-to-nearest-even).
  * Seed of tensor ``idx`` in workload ``wl`` is ``1000 * wl + idx`` with idx
    0 = q, 1 = k, 2 = v (linear-attention branch), 3 = q, 4 = k (window
    branch when it has its own q, k).
  * Decode step ``t`` draws q, k, v in that order from one generator seeded
    ``100000 + t``; a window decode step ``t`` draws its q, k (window dim)
    and v from one generator seeded ``200000 + t``.
  * The long-sequence workload multiplies raw k by ``outlier_scale`` at
    0-based positions ``p % outlier_every == outlier_every - 1`` before the
    bf16 rounding (exact in bf16 for a power of two).
"""
from __future__ import annotations

import dataclasses

import torch

DECODE_SEED_BASE = 100000
WINDOW_DECODE_SEED_BASE = 200000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int  # 1-based workload number used in the seed table
    dtype: str  # "f32" or "bf16"
    B: int
    H: int
    L: int
    d: int = 16  # Taylor feature (projected q/k) dim
    dv: int = 64
    scale: float = 1.0  # std of q, k, v
    chunk: int = 64
    eps: float = 1e-6
    # sliding-window branch (0 = none)
    window: int = 0
    d_qk: int = 0  # window-branch q/k dim (0 = shares the linear-attention q, k)
    swa_scale: float = 0.0
    # next-token steps after the prefill (0 = none)
    decode_steps: int = 0
    outlier_every: int = 0
    outlier_scale: float = 1.0
    description: str = ""

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def tol(self) -> float:
        """Max-abs-error bound as a multiple of the reference output RMS."""
        return 1e-4 if self.dtype == "f32" else 2e-2


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 1, "f32", B=1, H=1, L=256, dv=64, scale=1.0, window=64, d_qk=0,
        swa_scale=0.25,
        description="tiny causal BASED layer, fp32: Taylor linear attention + w=64 window, summed"),
    "prefill_360m": Workload(
        "prefill_360m", 2, "bf16", B=8, H=16, L=2048, dv=64, scale=0.5,
        description="BASED-360M-shaped prefill layer, bf16, chunk 64"),
    "decode_1p3b": Workload(
        "decode_1p3b", 3, "bf16", B=128, H=16, L=1024, dv=128, scale=1.0, decode_steps=1024,
        description="BASED-1.3B-shaped decode: 1024-token prefill then 1024 next-token steps"),
    "window_8k": Workload(
        "window_8k", 4, "bf16", B=4, H=16, L=8192, dv=64, scale=1.0, window=64, d_qk=64,
        swa_scale=1.0 / 8.0,
        description="w=64 sliding-window softmax (d=64) fused-added to Taylor linear attention"),
    "long_64k": Workload(
        "long_64k", 5, "bf16", B=1, H=16, L=65536, dv=64, scale=0.5, outlier_every=4096,
        outlier_scale=4.0,
        description="long-sequence chunked prefill with k outlier rows every 4096th position"),
    "window_decode_1p3b": Workload(
        "window_decode_1p3b", 6, "bf16", B=128, H=16, L=104, dv=128, scale=1.0, window=64, d_qk=64,
        swa_scale=1.0 / 8.0, decode_steps=1024,
        description="BASED-1.3B-shaped window next-token steps: w=64 ring filled from a 104-token "
                    "prefix, then 1024 steps"),
}


def randn(shape, seed: int, scale: float, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator("cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * scale
    return x.to(dtype)


def _outliers(k: torch.Tensor, wl: Workload) -> torch.Tensor:
    if wl.outlier_every:
        pos = torch.arange(k.shape[-2])
        sel = (pos % wl.outlier_every) == (wl.outlier_every - 1)
        k[..., sel, :] *= wl.outlier_scale
    return k


def linear_inputs(wl: Workload, B: int | None = None, H: int | None = None, L: int | None = None):
    """(q, k, v) for the Taylor linear-attention branch on the CPU.

    B, H, L may be reduced for a test; the draws are then those of the smaller
    shape (not a slice of the full-size draw).
    """
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    L = wl.L if L is None else L
    base = 1000 * wl.index
    q = randn((B, H, L, wl.d), base + 0, wl.scale, torch.float32)
    k = randn((B, H, L, wl.d), base + 1, wl.scale, torch.float32)
    v = randn((B, H, L, wl.dv), base + 2, wl.scale, torch.float32)
    k = _outliers(k, wl)
    dt = wl.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def window_inputs(wl: Workload, B: int | None = None, H: int | None = None, L: int | None = None):
    """(q, k) for the window branch; v is shared with the linear branch."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    L = wl.L if L is None else L
    base = 1000 * wl.index
    if wl.d_qk == 0:
        q, k, _ = linear_inputs(wl, B, H, L)
        return q, k
    q = randn((B, H, L, wl.d_qk), base + 3, wl.scale, wl.torch_dtype)
    k = randn((B, H, L, wl.d_qk), base + 4, wl.scale, wl.torch_dtype)
    return q, k


def decode_inputs(wl: Workload, t: int, B: int | None = None, H: int | None = None):
    """(q, k, v) for next-token step t: q,k [B,H,d], v [B,H,dv], N(0, scale^2)."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    g = torch.Generator("cpu").manual_seed(DECODE_SEED_BASE + int(t))
    q = torch.randn((B, H, wl.d), generator=g) * wl.scale
    k = torch.randn((B, H, wl.d), generator=g) * wl.scale
    v = torch.randn((B, H, wl.dv), generator=g) * wl.scale
    dt = wl.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def window_decode_inputs(wl: Workload, t: int, B: int | None = None, H: int | None = None):
    """(q, k, v) of window next-token step t: q,k [B,H,d_qk], v [B,H,dv]."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    g = torch.Generator("cpu").manual_seed(WINDOW_DECODE_SEED_BASE + int(t))
    q = torch.randn((B, H, wl.d_qk), generator=g) * wl.scale
    k = torch.randn((B, H, wl.d_qk), generator=g) * wl.scale
    v = torch.randn((B, H, wl.dv), generator=g) * wl.scale
    dt = wl.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def custom(shape_qk, shape_v, seed: int, scale: float = 1.0, dtype=torch.bfloat16):
    """(q, k, v) of arbitrary shapes for edge-case tests (seeds seed, seed+1, seed+2)."""
    q = randn(shape_qk, seed, scale, dtype)
    k = randn(shape_qk, seed + 1, scale, dtype)
    v = randn(shape_v, seed + 2, scale, dtype)
    return q, k, v
