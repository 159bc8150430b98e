"""Parity of the standalone in-place RoPE kernel against the oracle's fp64 rotation."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, max_abs, to_dev, values

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,tol", [("f32", 2e-6), ("bf16", BF16_TOL)])
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("D", [16, 64, 128, 576])
def test_rope_apply_positions(dtype, tol, interleaved, D):
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, S, N = 2, 37, 3
    x = synth.normal(500 + D, 0, (B, S, N, D), dtype)
    pos = np.random.default_rng(D).integers(0, 131072, (B, S)).astype(np.int32)
    xd = to_dev(x, dtype)
    attn.rope_apply_(xd, theta=5e5, positions=torch.as_tensor(pos, device="cuda"), interleaved=interleaved)
    want = oracle.rope_rotate(values(x, dtype), pos, 5e5, interleaved=interleaved)
    assert max_abs(xd.float().cpu().numpy(), want) <= tol


def test_rope_apply_default_positions():
    import causal_head_attention_gqa_amd as attn
    x = synth.normal(520, 0, (3, 50, 4, 128), "bf16")
    xd = to_dev(x, "bf16")
    attn.rope_apply_(xd, theta=1e4)
    want = oracle.rope_rotate(values(x, "bf16"), np.arange(50), 1e4)
    assert max_abs(xd.float().cpu().numpy(), want) <= BF16_TOL
