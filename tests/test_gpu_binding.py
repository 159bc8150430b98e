"""The binding refuses caller-supplied buffers that do not match what the kernels write (GPU only):
a wrong-shaped, wrong-dtype or strided `out` raises before anything is launched, and the given
buffer is left untouched."""
import pytest

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_reject_bad_out():
    import torch
    import causal_head_attention_gqa_amd as attn
    dev = "cuda"
    q = torch.randn((1, 40, 4, 64), device=dev).to(torch.bfloat16)
    kv = torch.randn((1, 40, 2, 64), device=dev).to(torch.bfloat16)
    small = torch.full((1, 20, 4, 64), 7.0, device=dev, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.prefill(q, kv, kv, out=small)
    assert bool((small == 7.0).all())
    with pytest.raises(TypeError):
        attn.prefill(q, kv, kv, out=torch.empty((1, 40, 4, 64), device=dev, dtype=torch.float32))
    with pytest.raises(ValueError):
        attn.prefill(q, kv, kv, out=torch.empty((1, 40, 64, 4), device=dev, dtype=torch.bfloat16).transpose(2, 3))
    dq = torch.randn((2, 4, 64), device=dev).to(torch.bfloat16)
    kc = torch.randn((2, 50, 2, 64), device=dev).to(torch.bfloat16)
    ctx = torch.tensor([50, 3], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        attn.decode(dq, kc, kc, ctx, out=torch.empty((2, 4, 32), device=dev, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        attn.decode(dq, kc, kc, ctx, workspace=torch.empty(1 << 20, dtype=torch.uint8))  # host memory
    good = attn.decode(dq, kc, kc, ctx, out=torch.empty((2, 4, 64), device=dev, dtype=torch.bfloat16))
    assert good.shape == (2, 4, 64)
