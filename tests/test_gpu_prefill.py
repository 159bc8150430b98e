"""Parity of the HIP prefill path against the fp64 oracle (GPU only).

Small cases span several 64-key tiles, every head-packing variant (MHA, GQA groups of 2/3/4,
MQA), ragged tails and the non-causal form, and are compared element by element over the whole
output. The two full-size workloads are checked in full (GPT-2-small shape) or on sampled rows
the oracle computes one by one (Llama-3-8B shape), in the same launch configuration the
benchmark times.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, F32_TOL, max_abs, to_dev, to_host_f64, values

pytestmark = pytest.mark.gpu


def _run(B, S, Nh, Nkv, D, dtype, rope, causal, wid, scale=None):
    import causal_head_attention_gqa_amd as attn
    q = synth.normal(wid, 0, (B, S, Nh, D), dtype)
    k = synth.normal(wid, 1, (B, S, Nkv, D), dtype)
    v = synth.normal(wid, 2, (B, S, Nkv, D), dtype)
    out = attn.prefill(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), rope_theta=rope, causal=causal,
                       scale=scale)
    got = to_host_f64(out)
    want = oracle.prefill(values(q, dtype), values(k, dtype), values(v, dtype), causal=causal, rope_theta=rope,
                          scale=scale)
    return got, want, (q, k, v)


SMALL_BF16 = [
    # B, S, Nh, Nkv, D, rope, causal
    (2, 200, 8, 2, 128, 5e5, True),    # GQA group 4, ragged tail
    (1, 333, 6, 6, 64, 0.0, True),     # MHA, 128-position work-groups
    (2, 130, 4, 2, 128, 1e4, True),    # GQA group 2
    (1, 97, 8, 1, 64, 1e4, True),      # MQA, two head groups per KV head
    (1, 150, 4, 1, 128, 0.0, False),   # full attention
    (3, 1, 4, 4, 64, 1e4, True),       # single token
    (1, 129, 12, 4, 64, 1e4, True),    # group of 3 -> one head per work-group
    (1, 64, 4, 2, 128, 0.0, True),     # exactly one tile
]


@pytest.mark.parametrize("case", SMALL_BF16, ids=lambda c: "B%dS%dH%dK%dD%d_r%g_c%d" % c)
def test_prefill_bf16_small(case):
    B, S, Nh, Nkv, D, rope, causal = case
    got, want, _ = _run(B, S, Nh, Nkv, D, "bf16", rope, causal, wid=100 + S)
    assert max_abs(got, want) <= BF16_TOL


GROWTH_CASES = [
    # B, S, Nh, Nkv, D, causal, scaled keys, factor: keys scaled after bf16 widening so that the
    # scores of those keys lie far above (or far below) those of the row's first 32-key block
    (1, 300, 8, 2, 128, True, (40, None), 20.0),   # later keys dominate: exact path, new reference
    (1, 300, 8, 2, 128, True, (0, 32), 20.0),      # the first block dominates: later p underflow
    (2, 200, 4, 4, 64, False, (100, None), 20.0),  # full attention
]


@pytest.mark.parametrize("case", GROWTH_CASES, ids=["later", "first", "full"])
def test_prefill_score_growth_beyond_reference(case):
    """The softmax reference max of a query is its first visible block's max; scores far above it
    send a block through the exact path (new reference, rescaled output). Compared with the oracle
    on inputs that do leave the fast path's range."""
    import causal_head_attention_gqa_amd as attn
    B, S, Nh, Nkv, D, causal, (k0, k1), factor = case
    wid = 180 + S
    q = synth.normal(wid, 0, (B, S, Nh, D), "bf16")
    kf = synth.as_f32(synth.normal(wid, 1, (B, S, Nkv, D), "bf16"), "bf16").copy()
    kf[:, k0:k1] *= factor
    k = synth.f32_to_bf16_bits(kf)
    v = synth.normal(wid, 2, (B, S, Nkv, D), "bf16")
    qv, kv, vv = values(q, "bf16"), values(k, "bf16"), values(v, "bf16")
    if k0 > 0:  # some query's later score exceeds its first block's max by more than 2^64
        G = Nh // Nkv
        sl = np.einsum("bshd,bthd->bhst", qv[:, :, ::G].astype(np.float64), kv.astype(np.float64))
        sl *= np.log2(np.e) / np.sqrt(D)
        assert np.any(sl[..., k0:].max(-1) > sl[..., :32].max(-1) + 64)
    out = attn.prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), causal=causal)
    got = to_host_f64(out)
    want = oracle.prefill(qv, kv, vv, causal=causal)
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= BF16_TOL


# Shapes the plain prefill sends to the split-key kernel (the usual grid is under two rounds of
# work-group slots and S >= 512): two waves share each 32-row query block and split its key tiles.
SPLITK_BF16 = [
    # B, S, Nh, Nkv, D, rope, causal
    (1, 600, 4, 4, 64, 0.0, True),     # MHA, ragged tail (600 = 18 x 32 + 24)
    (2, 512, 8, 2, 128, 5e5, True),    # GQA group 4, RoPE
    (1, 700, 6, 6, 64, 1e4, False),    # full attention, RoPE
    (1, 530, 4, 1, 128, 0.0, True),    # MQA, ragged tail
    (1, 545, 2, 2, 64, 1e4, True),     # a q-block with one wave's worth of tiles at the start
]


@pytest.mark.parametrize("case", SPLITK_BF16, ids=lambda c: "B%dS%dH%dK%dD%d_r%g_c%d" % c)
def test_prefill_split_key_kernel(case):
    B, S, Nh, Nkv, D, rope, causal = case
    got, want, _ = _run(B, S, Nh, Nkv, D, "bf16", rope, causal, wid=150 + S)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("k0,k1", [(40, None), (0, 32)], ids=["later", "first"])
def test_prefill_split_key_score_growth(k0, k1):
    """The split-key kernel's exact path: keys scaled so that later scores exceed a wave's first
    block's max by far (or fall far below it)."""
    import causal_head_attention_gqa_amd as attn
    B, S, Nh, Nkv, D = 1, 600, 4, 2, 128
    wid = 190
    q = synth.normal(wid, 0, (B, S, Nh, D), "bf16")
    kf = synth.as_f32(synth.normal(wid, 1, (B, S, Nkv, D), "bf16"), "bf16").copy()
    kf[:, k0:k1] *= 20.0
    k = synth.f32_to_bf16_bits(kf)
    v = synth.normal(wid, 2, (B, S, Nkv, D), "bf16")
    out = attn.prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"))
    got = to_host_f64(out)
    want = oracle.prefill(values(q, "bf16"), values(k, "bf16"), values(v, "bf16"))
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= BF16_TOL


def test_prefill_split_key_row0_is_v0_exactly():
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q = synth.normal(195, 0, (2, 640, 4, 64), "bf16")
    kv = synth.normal(195, 1, (2, 640, 4, 64), "bf16")
    vd = to_dev(synth.normal(195, 2, (2, 640, 4, 64), "bf16"), "bf16")
    out = attn.prefill(to_dev(q, "bf16"), to_dev(kv, "bf16"), vd, rope_theta=1e4)
    assert torch.equal(out[:, 0], vd[:, 0])


SMALL_F32 = [
    (1, 128, 4, 4, 16, 1e4, True),
    (2, 150, 4, 2, 32, 1e4, True),
    (1, 70, 8, 2, 64, 5e5, True),
    (1, 33, 2, 1, 16, 0.0, False),
]


@pytest.mark.parametrize("case", SMALL_F32, ids=lambda c: "B%dS%dH%dK%dD%d_r%g_c%d" % c)
def test_prefill_f32_small(case):
    B, S, Nh, Nkv, D, rope, causal = case
    got, want, _ = _run(B, S, Nh, Nkv, D, "f32", rope, causal, wid=200 + S)
    assert max_abs(got, want) <= F32_TOL


def test_tiny_f32_workload_full():
    """B=1, S=128, 4 heads of 16, fp32, RoPE 1e4: every output within 1e-5 of the oracle."""
    w = synth.TINY_F32
    got, want, _ = _run(w.B, w.S, w.Nh, w.Nkv, w.Dh, w.dtype, w.rope_theta, True, wid=w.wid)
    assert got.shape == (1, 128, 4, 16)
    assert max_abs(got, want) <= F32_TOL


def test_row0_is_v0_exactly():
    """Position 0 sees only itself: out[:, 0, h] equals v[:, 0, h // G] bit for bit."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q = synth.normal(300, 0, (2, 70, 8, 128), "bf16")
    k = synth.normal(300, 1, (2, 70, 2, 128), "bf16")
    v = synth.normal(300, 2, (2, 70, 2, 128), "bf16")
    vd = to_dev(v, "bf16")
    out = attn.prefill(to_dev(q, "bf16"), to_dev(k, "bf16"), vd, rope_theta=5e5)
    for h in range(8):
        assert torch.equal(out[:, 0, h], vd[:, 0, h // 4])


def test_scale_argument():
    got, want, _ = _run(1, 90, 4, 2, 64, "bf16", 0.0, True, wid=301, scale=0.3)
    assert max_abs(got, want) <= BF16_TOL


def test_causality_on_gpu():
    """Changing keys/values after position t leaves outputs up to t unchanged."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q = to_dev(synth.normal(302, 0, (1, 160, 4, 128), "bf16"), "bf16")
    k = to_dev(synth.normal(302, 1, (1, 160, 1, 128), "bf16"), "bf16")
    v = to_dev(synth.normal(302, 2, (1, 160, 1, 128), "bf16"), "bf16")
    a = attn.prefill(q, k, v, rope_theta=1e4)
    k2, v2 = k.clone(), v.clone()
    k2[:, 100:] = 3.0
    v2[:, 100:] = -7.0
    b = attn.prefill(q, k2, v2, rope_theta=1e4)
    assert torch.equal(a[:, :100], b[:, :100])
    assert not torch.equal(a[:, 100:], b[:, 100:])


def test_empty_batch_is_a_no_op():
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    q = torch.zeros((0, 16, 4, 64), dtype=torch.bfloat16, device="cuda")
    kv = q[:, :, :2].contiguous()
    out = attn.prefill(q, kv, kv)
    assert out.shape == q.shape


def test_gpt2_small_prefill_full():
    """B=8, S=1024, 12 heads of 64, bf16, no RoPE: all 6.3M outputs against the oracle."""
    w = synth.GPT2_PREFILL
    got, want, _ = _run(w.B, w.S, w.Nh, w.Nkv, w.Dh, w.dtype, w.rope_theta, True, wid=w.wid)
    assert max_abs(got, want) <= BF16_TOL


def test_llama3_prefill_every_head_sampled_rows():
    """B=4, S=8192, 32 query / 8 KV heads of 128, RoPE 5e5: the full launch on the GPU (XCD-major
    work-group order, heaviest q-tiles first), then EVERY (batch, query head) pair on at least 256
    rows against the oracle: the edge rows of the 32-row work-group tiles and 32-key blocks (0, 1,
    31, 32, 33, 63, 64, 127, 128, the middle, the last tiles) plus rows drawn per pair. The oracle
    does ~1 GFLOP per pair (~20 s in all); the whole 4.4 TFLOP output would take hours on the host.
    Over the whole output: every element is written (a NaN fill is gone everywhere), and row 0 of
    every head, a softmax over a single key, is that key's value row exactly."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    w = synth.LLAMA3_PREFILL
    q, k, v = w.inputs()
    qd, vd = to_dev(q, "bf16"), to_dev(v, "bf16")
    out = attn.prefill(qd, to_dev(k, "bf16"), vd, rope_theta=w.rope_theta, out=torch.full_like(qd, float("nan")))
    assert bool(torch.isfinite(out).all())
    for h in range(w.Nh):
        assert torch.equal(out[:, 0, h], vd[:, 0, h // (w.Nh // w.Nkv)])
    edges = np.array([0, 1, 31, 32, 33, 63, 64, 127, 128, 4095, 4096, 8127, 8128, 8159, 8160, 8190, 8191])
    rng = np.random.default_rng(7)
    worst, n_rows = 0.0, 0
    qv, kv, vv = values(q, "bf16"), values(k, "bf16"), values(v, "bf16")
    for b in range(w.B):
        for h in range(w.Nh):
            rows = np.unique(np.concatenate([edges, rng.choice(w.S, 300, replace=False)]))
            assert len(rows) >= 256
            got = out[b, torch.as_tensor(rows, device=out.device), h].float().cpu().numpy()
            want = oracle.prefill_rows(qv, kv, vv, b, h, rows, rope_theta=w.rope_theta)
            err = max_abs(got, want)
            assert err <= BF16_TOL, (b, h, err)
            worst = max(worst, err)
            n_rows += len(rows)
    assert n_rows >= w.B * w.Nh * 256


@pytest.mark.parametrize("B,S,Nh,Nkv,rope", [(4, 2048, 32, 8, 5e5), (2, 400, 32, 8, 0.0), (3, 300, 12, 3, 1e4)],
                         ids=["llama-2048-rope", "32-pairs-400", "9-pairs-rope"])
def test_work_lists_give_the_static_order_bits(B, S, Nh, Nkv, rope):
    """The work lists' counters at the end of the workspace only change which work-group computes a
    q-tile (and let fast XCDs take items from slow ones): the output equals, bit for bit, that of a
    call whose workspace stops short of them (and, without RoPE, of a call with no workspace), on
    two calls in a row (the counters are zeroed by each call). 9 pairs do not split over the XCDs:
    no lists there. Shapes that take the one-item-per-work-group kernel, not the split-key one."""
    import ctypes
    import causal_head_attention_gqa_amd as attn
    from causal_head_attention_gqa_amd import lib
    torch = __import__("torch")
    wid = 720 + S
    q = to_dev(synth.normal(wid, 0, (B, S, Nh, 128), "bf16"), "bf16")
    k = to_dev(synth.normal(wid, 1, (B, S, Nkv, 128), "bf16"), "bf16")
    v = to_dev(synth.normal(wid, 2, (B, S, Nkv, 128), "bf16"), "bf16")
    full = attn.prefill_workspace_bytes(B, S, Nkv, 128, rope, attn.ATTN_BF16)
    # the workspace sits at the start of a larger buffer whose tail holds a canary: nothing past the
    # figure may be written
    buf = torch.full((full + 4096,), 0xA5, dtype=torch.uint8, device="cuda")

    def call(ws_ptr, ws_len):
        out = torch.full_like(q, float("nan"))
        st = attn.load().attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, Nh, Nkv, 128,
                                      ctypes.c_float(rope), 1, ctypes.c_float(0.0), attn.ATTN_BF16, ws_ptr,
                                      ctypes.c_size_t(ws_len), lib._stream_ptr(q.device))
        assert st == 0
        torch.cuda.synchronize()
        return out

    listed = call(buf.data_ptr(), full)
    assert bool((buf[full:] == 0xA5).all())
    static = call(buf.data_ptr(), full - 512)
    assert torch.isfinite(listed.float()).all()
    assert torch.equal(listed, static)
    assert torch.equal(call(buf.data_ptr(), full), static)
    assert bool((buf[full:] == 0xA5).all())
    if rope == 0.0:
        assert torch.equal(call(None, 0), static)
