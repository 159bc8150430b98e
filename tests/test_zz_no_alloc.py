"""attn_decode_noalloc (no workspace: the library's static per-GPU scratch holds the split
partials) against attn_decode on the same inputs (GPU only).

Both calls run the same kernels with the same chunk plan, so the outputs must be bit-identical.
Two calls in a row, the second on a smaller input, check that the scratch left by the first call
does not leak into the second; an oversized request is refused before anything is launched.
"""
import math

import numpy as np
import pytest

import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _case(wid, B, Nh, Nkv, Dqk, Dv, T, mla):
    torch = __import__("torch")
    rng = np.random.default_rng(wid)
    ctx = rng.integers(1, T, size=B, endpoint=True).astype(np.int32)
    ctx[0] = T
    q = to_dev(synth.normal(wid, 0, (B, Nh, Dqk), "bf16"), "bf16")
    kc = to_dev(synth.normal(wid, 1, (B, T, Nkv, Dqk), "bf16"), "bf16")
    vc = kc[..., :Dv] if mla else to_dev(synth.normal(wid, 2, (B, T, Nkv, Dv), "bf16"), "bf16")
    return q, kc, vc, torch.as_tensor(ctx, device="cuda")


CASES = [
    # (first call), (second, smaller call): B, Nh, Nkv, Dqk, Dv, T, mla, scale, rope
    ((64, 32, 8, 128, 128, 4096, False, None, 0.0), (5, 32, 8, 128, 128, 700, False, None, 5e5)),
    ((32, 128, 1, 576, 512, 4096, True, 1 / math.sqrt(192), 0.0), (3, 64, 1, 576, 512, 900, True,
                                                                    1 / math.sqrt(192), 1e4)),
]


@pytest.mark.parametrize("first,second", CASES, ids=["gqa", "mla"])
def test_noalloc_matches_decode_twice(first, second):
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    for i, (B, Nh, Nkv, Dqk, Dv, T, mla, scale, rope) in enumerate((first, second)):
        q, kc, vc, ctx = _case(800 + 10 * i + int(mla), B, Nh, Nkv, Dqk, Dv, T, mla)
        want = attn.decode(q, kc, vc, ctx, scale=scale, rope_theta=rope)
        got = torch.full_like(want, float("nan"))
        attn.decode_noalloc(q, kc, vc, ctx, scale=scale, rope_theta=rope, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (i, B, Nh, mla)


def test_noalloc_refuses_requests_beyond_the_scratch():
    import causal_head_attention_gqa_amd as attn
    lib = attn.load()
    cap = attn.decode_noalloc_max_bytes()
    assert cap == 64 << 20
    # 4096 sequences x 32 heads x 8 chunks of 1024 tokens of bf16 partials: far beyond 64 MiB
    need = attn.decode_workspace_bytes(4096, 32, 8, 128, 128, 8192, attn.ATTN_BF16)
    assert need > cap
    st = lib.attn_decode_noalloc(16, 16, 16, 16, 16, 4096, 32, 8, 128, 128, 8192, 128, 128, 0.0, 0.0,
                                 attn.ATTN_BF16, None)
    assert st == 3  # ATTN_ERR_WORKSPACE, returned before any launch
