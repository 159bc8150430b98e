"""Parity of MLA's non-absorbed prefill (q/k head dim 192 = 128 + 64 decoupled RoPE dims, v and
out head dim 128) against the fp64 oracle (GPU only).

Small cases cover the three head packings (1, 2 or 4 query heads per KV head), ragged tails, a
single token and the non-causal form, element by element. The DeepSeek-V3-shaped workload
(B=1, S=4096, 128 heads) is checked on sampled rows that the oracle computes one by one.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, max_abs, to_dev, to_host_f64, values

pytestmark = pytest.mark.gpu


def _inputs(wid, B, S, Nh, Nkv):
    q = synth.normal(wid, 0, (B, S, Nh, 192), "bf16")
    k = synth.normal(wid, 1, (B, S, Nkv, 192), "bf16")
    v = synth.normal(wid, 2, (B, S, Nkv, 128), "bf16")
    return q, k, v


SMALL = [
    # B, S, Nh, Nkv, rope, causal
    (1, 200, 4, 4, 1e4, True),     # one query head per KV head (DeepSeek's per-head K/V), ragged
    (2, 97, 4, 4, 1e4, True),      # two sequences, tail inside the first tile
    (1, 130, 8, 2, 1e4, True),     # four query heads per KV head
    (1, 150, 4, 2, 0.0, False),    # two per KV head, full attention, no RoPE
    (3, 1, 4, 4, 1e4, True),       # single token
    (1, 256, 2, 2, 1e4, True),     # whole 128-position work-groups, no tail
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%dS%dH%dK%d_r%g_c%d" % c)
def test_mla_prefill_small(case):
    import causal_head_attention_gqa_amd as attn
    B, S, Nh, Nkv, rope, causal = case
    q, k, v = _inputs(600 + S, B, S, Nh, Nkv)
    out = attn.prefill_mla(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), rope_theta=rope,
                           causal=causal)
    assert tuple(out.shape) == (B, S, Nh, 128)
    want = oracle.prefill(values(q, "bf16"), values(k, "bf16"), values(v, "bf16"), causal=causal,
                          rope_theta=rope)
    assert max_abs(to_host_f64(out), want) <= BF16_TOL


def test_mla_prefill_row0_is_v0_exactly():
    """Position 0 sees only its own key, whatever the rotation: out[:, 0, h] == v[:, 0, h // G]."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q, k, v = _inputs(650, 2, 70, 8, 4)
    vd = to_dev(v, "bf16")
    out = attn.prefill_mla(to_dev(q, "bf16"), to_dev(k, "bf16"), vd, rope_theta=1e4)
    assert torch.equal(out[:, 0], vd[:, 0].repeat_interleave(2, dim=1))


def test_mla_prefill_scale_and_workspace_reuse():
    """A caller-owned workspace of the queried size gives the same bits as one the binding
    allocates. An explicit scale of 1/sqrt(192) matches the default within the tolerance (the
    explicit value is an fp32 number, the default is formed in fp64, so the two can differ in the
    last bit of the exponent scale and hence in a few output bits)."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q, k, v = _inputs(651, 1, 160, 4, 4)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a = attn.prefill_mla(qd, kd, vd, rope_theta=1e4)
    ws = torch.empty(attn.prefill_mla_workspace_bytes(1, 160, 4, 1e4), dtype=torch.uint8, device=qd.device)
    c = attn.prefill_mla(qd, kd, vd, rope_theta=1e4, workspace=ws)
    assert torch.equal(a, c), "caller workspace changed the result"
    b = attn.prefill_mla(qd, kd, vd, rope_theta=1e4, scale=1.0 / np.sqrt(192.0))
    want = oracle.prefill(values(q, "bf16"), values(k, "bf16"), values(v, "bf16"), causal=True, rope_theta=1e4)
    assert max_abs(to_host_f64(b), want) <= BF16_TOL
    assert max_abs(to_host_f64(a), to_host_f64(b)) <= 2 ** -6
    k_before = kd.clone()
    attn.prefill_mla(qd, kd, vd, rope_theta=1e4)
    assert torch.equal(kd, k_before)  # keys are rotated into the workspace, never in place


def test_mla_prefill_full_size_sampled_rows():
    """DeepSeek-V3-shaped non-absorbed prefill (B=1, S=4096, 128 heads, 192/128, RoPE 1e4) in the
    benchmark's launch configuration; sampled (head, row) outputs against the oracle."""
    import causal_head_attention_gqa_amd as attn
    w = synth.MLA_PREFILL
    q, k, v = w.inputs()
    out = to_host_f64(attn.prefill_mla(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                       rope_theta=w.rope_theta))
    assert out.shape == (w.B, w.S, w.Nh, w.dv)
    qv, kv, vv = values(q, "bf16"), values(k, "bf16"), values(v, "bf16")
    rng = np.random.default_rng(6)
    heads = [0, 1, 63, 127] + list(rng.integers(0, w.Nh, 4))
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, 2047, 4095], rng.integers(0, w.S, 8)]))
    for h in heads:
        want = oracle.prefill_rows(qv, kv, vv, 0, int(h), rows, rope_theta=w.rope_theta)
        assert max_abs(out[0, rows, h], want) <= BF16_TOL, h


def test_mla_prefill_work_lists_give_the_static_order_bits():
    """The optional work-list counters at the end of the workspace only change which work-group takes
    a q-tile: the output equals, bit for bit, that of a call whose workspace stops short of them
    (64 (sequence, head) pairs: one list per XCD)."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, S, Nh, Nkv, rope = 2, 600, 32, 32, 1e4
    q, k, v = (to_dev(t, "bf16") for t in _inputs(640, B, S, Nh, Nkv))
    full = attn.prefill_mla_workspace_bytes(B, S, Nkv, rope)
    buf = torch.full((full + 4096,), 0xA5, dtype=torch.uint8, device="cuda")  # canary past the figure
    listed = attn.prefill_mla(q, k, v, rope_theta=rope, workspace=buf[:full])
    torch.cuda.synchronize()
    assert bool((buf[full:] == 0xA5).all())
    static = attn.prefill_mla(q, k, v, rope_theta=rope, workspace=buf[:full - 512])
    assert torch.isfinite(listed.float()).all()
    assert torch.equal(listed, static)
