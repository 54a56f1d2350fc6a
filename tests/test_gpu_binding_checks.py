"""The Python binding rejects caller-supplied tensors whose shape, device or
dtype does not match the call, before anything is launched (an undersized
output or state would otherwise be written past its end by the kernels)."""
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def based():
    import linear_attention_sequence_taylor_amd as based  # fails loudly without the .so

    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return based


def _bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device=DEV)


def _f32(*shape):
    return torch.zeros(shape, dtype=torch.float32, device=DEV)


B, H, L, D, DV = 2, 3, 70, 16, 64
F = 1 + D + D * D


def test_prefill_output_shapes(based):
    q, k, v = _bf16(B, H, L, D), _bf16(B, H, L, D), _bf16(B, H, L, DV)
    with pytest.raises(ValueError, match="y must have shape"):
        based.based_prefill(q, k, v, y=_f32(B, H, L - 1, DV))
    with pytest.raises(ValueError, match="S must have shape"):
        based.based_prefill(q, k, v, S=_f32(B, H, F - 1, DV))
    with pytest.raises(ValueError, match="z must have shape"):
        based.based_prefill(q, k, v, z=_f32(B, H * F))
    with pytest.raises(ValueError, match="initial_state must have shapes"):
        based.based_prefill(q, k, v, initial_state=(_f32(F, DV), _f32(B, H, F)))
    # (this shape's launch plan uses no workspace at all)
    with pytest.raises(ValueError, match="workspace must be on"):
        based.based_prefill(q, k, v, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="v must be on"):
        based.based_prefill(q, k, v.cpu())


def test_hybrid_output_shapes(based):
    q, k, v = _bf16(B, H, L, D), _bf16(B, H, L, D), _bf16(B, H, L, DV)
    qw, kw = _bf16(B, H, L, 64), _bf16(B, H, L, 64)
    with pytest.raises(ValueError, match="y must have shape"):
        based.based_hybrid_prefill(q, k, qw, kw, v, y=_f32(B, H, L, DV + 1))
    with pytest.raises(ValueError, match="S must have shape"):
        based.based_hybrid_prefill(q, k, qw, kw, v, S=_f32(B, H, F, DV // 2))


def test_decode_state_shapes(based):
    q, k, v = _bf16(B, H, D), _bf16(B, H, D), _bf16(B, H, 128)
    S, z = _f32(B, H, F, 128), _f32(B, H, F)
    with pytest.raises(ValueError, match="S must have shape"):
        based.based_decode_step(q, k, v, _f32(B, H, F, 64), z)
    with pytest.raises(ValueError, match="z must have shape"):
        based.based_decode_step(q, k, v, S, _f32(B, H, F - 1))
    with pytest.raises(ValueError, match="shape mismatch"):
        based.based_decode_step(q, _bf16(B, H - 1, D), v, S, z)
    with pytest.raises(ValueError, match="y must have shape"):
        based.based_decode_step(q, k, v, S, z, y=_f32(B, H, 64))


def test_window_shapes(based):
    q, k, v = _bf16(B, H, L, 64), _bf16(B, H, L, 64), _bf16(B, H, L, DV)
    with pytest.raises(ValueError, match="shape mismatch"):
        based.swa_forward(q, _bf16(B, H, L - 5, 64), v)
    with pytest.raises(ValueError, match="add must have shape"):
        based.swa_forward(q, k, v, add=_f32(B, H, L, DV // 2))
    kc, vc = based.swa_cache_fill(k, v, window=64)
    pos = torch.full((B,), L, dtype=torch.int64, device=DEV)
    with pytest.raises(ValueError, match="y must have shape"):
        based.swa_decode_step(_bf16(B, H, 64), _bf16(B, H, 64), _bf16(B, H, DV), kc, vc, pos, y=_f32(B, H, 1))
    with pytest.raises(ValueError, match="shape mismatch"):
        based.swa_cache_fill(k, _bf16(B, H, L - 1, DV), window=64)


def test_backward_output_shapes(based):
    q, k, v = _bf16(B, H, L, D), _bf16(B, H, L, D), _bf16(B, H, L, DV)
    dy = _f32(B, H, L, DV)
    with pytest.raises(ValueError, match="dq must have shape"):
        based.based_prefill_backward(q, k, v, dy, dq=_f32(B, H, L, 8))
    with pytest.raises(ValueError, match="dv must have shape"):
        based.based_prefill_backward(q, k, v, dy, dv=_f32(B, H, L - 1, DV))
    # a host workspace must be refused by the binding; it is also too small,
    # so should that check ever let it through, the library's size check
    # refuses the call before any launch
    with pytest.raises(ValueError, match="workspace must be on"):
        based.based_prefill_backward(q, k, v, dy, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(based.BasedError):
        based.based_prefill_backward(q, k, v, dy, workspace=torch.zeros(16, dtype=torch.uint8, device=DEV))


def test_valid_calls_still_run(based):
    """The same calls with matching tensors go through (outputs supplied)."""
    q, k, v = _bf16(B, H, L, D), _bf16(B, H, L, D), _bf16(B, H, L, DV)
    y, S, z = _f32(B, H, L, DV), _f32(B, H, F, DV), _f32(B, H, F)
    based.based_prefill(q, k, v, y=y, S=S, z=z, initial_state=(S, z))
    based.based_prefill_backward(q, k, v, _f32(B, H, L, DV), dq=_f32(B, H, L, D), dk=_f32(B, H, L, D),
                                 dv=_f32(B, H, L, DV))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
