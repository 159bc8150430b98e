"""Parity of the HIP KV-cache decode paths (GQA split-KV and MLA-absorbed) against the oracle.

Small cases cover MHA/GQA/MQA groups, context lengths that end inside a chunk, a context of
one key, and RoPE applied to the query in-kernel. The full Llama-3-8B-shaped decode (B=64,
contexts drawn in [1024, 8192]) and the full MLA-absorbed decode (B=32, 128 heads, 576-dim
shared row, context 4096) are compared over every output. Cache rows beyond a sequence's
context are filled with NaN in one test to show they are never read.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, max_abs, to_dev, values

pytestmark = pytest.mark.gpu


def _oracle_decode(q, kc, vc, ctx, scale=None, rope=0.0, mla=False):
    """Per-sequence oracle calls on fp64 slices (keeps host memory and time bounded)."""
    B, Nh, _ = q.shape
    Dv = 512 if mla else vc.shape[3]
    out = np.empty((B, Nh, Dv))
    for b in range(B):
        c = int(ctx[b])
        kb = values(kc[b:b + 1, :c], "bf16").astype(np.float64)
        vb = kb[..., :Dv] if mla else values(vc[b:b + 1, :c], "bf16").astype(np.float64)
        out[b] = oracle.decode(values(q[b:b + 1], "bf16"), kb, vb, np.array([c]), scale=scale, rope_theta=rope)[0]
    return out


def _gpu_decode(q, kc, vc, ctx, scale=None, rope=0.0, mla=False):
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    kd = to_dev(kc, "bf16")
    vd = kd[..., :512] if mla else to_dev(vc, "bf16")
    ctx_d = torch.as_tensor(np.asarray(ctx, np.int32), device="cuda")
    out = attn.decode(to_dev(q, "bf16"), kd, vd, ctx_d, scale=scale, rope_theta=rope)
    return out.float().cpu().numpy()


GQA_CASES = [
    # B, Nh, Nkv, D, max_ctx, ctx list (None: random in [1, max_ctx]), rope
    (3, 32, 8, 128, 1500, [1, 777, 1500], 0.0),
    (4, 8, 8, 128, 600, None, 0.0),       # MHA
    (2, 16, 2, 64, 2049, [2049, 513], 0.0),  # group of 8
    (5, 12, 1, 128, 300, None, 0.0),      # MQA with 12 heads: one group of 12
    (2, 32, 1, 128, 700, [700, 129], 0.0),  # MQA with 32 heads: two groups of 16 per KV head
    (2, 64, 2, 64, 520, [520, 300], 1e4),   # 32 query heads per KV head, RoPE
    (2, 32, 8, 128, 900, [900, 17], 5e5),  # q rotated at ctx-1
    (3, 6, 2, 64, 100, [1, 2, 64], 1e4),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: "B%dH%dK%dD%dT%d" % c[:5])
def test_decode_gqa_small(case):
    B, Nh, Nkv, D, T, ctx, rope = case
    wid = 400 + T
    rng = np.random.default_rng(wid)
    ctx = np.asarray(ctx if ctx is not None else rng.integers(1, T, B, endpoint=True), np.int32)
    q = synth.normal(wid, 0, (B, Nh, D), "bf16")
    kc = synth.normal(wid, 1, (B, T, Nkv, D), "bf16")
    vc = synth.normal(wid, 2, (B, T, Nkv, D), "bf16")
    got = _gpu_decode(q, kc, vc, ctx, rope=rope)
    want = _oracle_decode(q, kc, vc, ctx, rope=rope)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("D", [64, 128])
def test_decode_contexts_at_chunk_edges(D):
    """64 sequences x 8 KV heads (Dh 64 and 128): the plan splits contexts into 1024-token chunks;
    contexts of 1, at, just below and just above the chunk edges (one key into a new chunk), and at
    quarter-chunk edges, against the oracle."""
    B, Nh, Nkv, T = 64, 8, 8, 2049
    edges = [1, 2, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048, 2049]
    ctx = np.array([edges[i % len(edges)] for i in range(B)], np.int32)
    q = synth.normal(560 + D, 0, (B, Nh, D), "bf16")
    kc = synth.normal(560 + D, 1, (B, T, Nkv, D), "bf16")
    vc = synth.normal(560 + D, 2, (B, T, Nkv, D), "bf16")
    got = _gpu_decode(q, kc, vc, ctx)
    pick = np.arange(len(edges))  # one sequence per context length
    want = _oracle_decode(q[pick], kc[pick], vc[pick], ctx[pick])
    assert max_abs(got[pick], want) <= BF16_TOL


@pytest.mark.parametrize("D", [64, 128])
def test_decode_more_than_64_sequences(D):
    """130 sequences x 8 KV heads (Dh 64 and 128) with contexts up to 1100: 1024-token chunks, so the
    kernel's work-item order (every full chunk, then the short last chunks) spans three blocks of 64
    sequences in both parts; sequences from each block against the oracle."""
    B, Nh, Nkv, T = 130, 8, 8, 1100
    rng = np.random.default_rng(575)
    ctx = rng.integers(1, T, B, endpoint=True).astype(np.int32)
    ctx[[5, 70, 129]] = [1024, 1100, 1025]
    q = synth.normal(575, 0, (B, Nh, D), "bf16")
    kc = synth.normal(575, 1, (B, T, Nkv, D), "bf16")
    vc = synth.normal(575, 2, (B, T, Nkv, D), "bf16")
    got = _gpu_decode(q, kc, vc, ctx)
    pick = np.array([0, 5, 63, 64, 70, 100, 127, 128, 129])
    want = _oracle_decode(q[pick], kc[pick], vc[pick], ctx[pick])
    assert max_abs(got[pick], want) <= BF16_TOL


def test_decode_workspace_needs_no_clearing():
    """The split partials live in the caller's workspace: a workspace holding arbitrary bytes, and the
    same workspace reused by consecutive calls with other contexts (and so other chunk counts), give
    the oracle's result every time."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, Nh, Nkv, D, T = 6, 16, 4, 128, 3000
    q = synth.normal(570, 0, (B, Nh, D), "bf16")
    kc = synth.normal(570, 1, (B, T, Nkv, D), "bf16")
    vc = synth.normal(570, 2, (B, T, Nkv, D), "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
    need = attn.decode_workspace_bytes(B, Nh, Nkv, D, D, T, attn.ATTN_BF16)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(570)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda", generator=gen)
    contexts = [[3000, 1, 2048, 1025, 999, 2500], [17, 3000, 3000, 2049, 64, 1], [3000, 1, 2048, 1025, 999, 2500]]
    for i, ctx in enumerate(contexts):
        if i == 2:
            ws.fill_(0xFF)
        ctx = np.asarray(ctx, np.int32)
        out = attn.decode(qd, kd, vd, torch.as_tensor(ctx, device="cuda"), workspace=ws)
        got = out.float().cpu().numpy()
        assert max_abs(got, _oracle_decode(q, kc, vc, ctx)) <= BF16_TOL, f"call {i}"


@pytest.mark.parametrize("Nkv", [2, 4])
def test_decode_never_reads_beyond_context(Nkv):
    B, Nh, D, T = 3, 8, 128, 700
    ctx = np.array([5, 333, 700], np.int32)
    q = synth.normal(450, 0, (B, Nh, D), "bf16")
    kc = synth.normal(450, 1, (B, T, Nkv, D), "bf16")
    vc = synth.normal(450, 2, (B, T, Nkv, D), "bf16")
    clean = _gpu_decode(q, kc, vc, ctx)
    kn, vn = kc.copy(), vc.copy()
    for b, c in enumerate(ctx):
        kn[b, c:] = 0x7FC0  # bf16 NaN
        vn[b, c:] = 0x7FC0
    dirty = _gpu_decode(q, kn, vn, ctx)
    assert np.all(np.isfinite(dirty))
    assert np.array_equal(clean, dirty)


def test_mla_decode_small():
    B, Nh, T = 2, 32, 300
    ctx = np.array([300, 45], np.int32)
    q = synth.normal(460, 0, (B, Nh, 576), "bf16")
    kc = synth.normal(460, 1, (B, T, 1, 576), "bf16")
    scale = 1.0 / math.sqrt(192)
    got = _gpu_decode(q, kc, None, ctx, scale=scale, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=scale, mla=True)
    assert max_abs(got, want) <= BF16_TOL


def test_mla_decode_decoupled_rope():
    """q^R (dims 512..575) rotated in-kernel at ctx-1; the cache rows hold rotated k^R."""
    B, Nh, T = 2, 32, 200
    ctx = np.array([200, 77], np.int32)
    q = synth.normal(470, 0, (B, Nh, 576), "bf16")
    kc = synth.normal(470, 1, (B, T, 1, 576), "bf16")
    scale = 1.0 / math.sqrt(192)
    got = _gpu_decode(q, kc, None, ctx, scale=scale, rope=1e4, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=scale, rope=1e4, mla=True)
    assert max_abs(got, want) <= BF16_TOL


MLA_PAIR_CASES = [
    # B, Nh, max_ctx, ctx list, rope: head counts that are multiples of 64 (pairs of waves sharing
    # 32 heads); contexts of one token, ending inside a 32-token tile, and splits left empty
    (3, 128, 1000, [1000, 45, 1], 0.0),
    (2, 64, 333, [333, 32], 0.0),
    (2, 64, 200, [200, 77], 1e4),      # decoupled q^R RoPE (held by the upper reduction half)
    (2, 192, 130, [130, 96], 5e5),     # three head groups
    # multiples of 128: one work-group holds all heads of a row (64 per wave pair)
    (9, 128, 700, [700, 1, 33, 64, 65, 512, 513, 95, 640], 0.0),  # grid with empty ids (B % 8 != 0)
    (2, 256, 333, [333, 32], 0.0),     # two 128-head groups
    (2, 128, 200, [200, 77], 1e4),     # q^R rotated in-kernel, with its bf16 residual products
    (9, 128, 700, [700, 1, 33, 64, 65, 512, 513, 95, 640], 1e4),
    (2, 256, 333, [333, 32], 5e5),
]


@pytest.mark.parametrize("case", MLA_PAIR_CASES, ids=lambda c: "B%dH%dT%d" % c[:3])
def test_mla_decode_head_pairs(case):
    B, Nh, T, ctx, rope = case
    wid = 480 + T
    ctx = np.asarray(ctx, np.int32)
    q = synth.normal(wid, 0, (B, Nh, 576), "bf16")
    kc = synth.normal(wid, 1, (B, T, 1, 576), "bf16")
    scale = 1.0 / math.sqrt(192)
    got = _gpu_decode(q, kc, None, ctx, scale=scale, rope=rope, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=scale, rope=rope, mla=True)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("Nh", [64, 128])
def test_mla_decode_single_chunk(Nh):
    """Enough (sequence, head group) units that each sequence is one chunk: the kernel writes the
    normalised output itself (no split partials, no merge), so the call needs no workspace: the C
    entry point is called with a NULL one and matches the oracle."""
    import ctypes
    import causal_head_attention_gqa_amd as attn
    from causal_head_attention_gqa_amd import lib
    torch = __import__("torch")
    B, T = 256, 64
    rng = np.random.default_rng(490)
    ctx = rng.integers(1, T, B, endpoint=True).astype(np.int32)
    q = synth.normal(490, 0, (B, Nh, 576), "bf16")
    kc = synth.normal(490, 1, (B, T, 1, 576), "bf16")
    scale = 1.0 / math.sqrt(192)
    assert attn.decode_workspace_bytes(B, Nh, 1, 576, 512, T, attn.ATTN_BF16) == 0
    qd, kd = to_dev(q, "bf16"), to_dev(kc, "bf16")
    cd = torch.as_tensor(ctx, device="cuda")
    out = torch.full((B, Nh, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = attn.load().attn_decode(qd.data_ptr(), kd.data_ptr(), kd.data_ptr(), cd.data_ptr(), out.data_ptr(), B, Nh, 1,
                                 576, 512, T, 576, 576, ctypes.c_float(0.0), ctypes.c_float(scale), attn.ATTN_BF16,
                                 None, 0, lib._stream_ptr(qd.device))
    assert st == 0
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    want = _oracle_decode(q, kc, None, ctx, scale=scale, mla=True)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("B,T,ctx,rope,Nh", [(2, 300, [300, 200], 0.0, 64), (2, 300, [300, 260], 1e4, 64),
                                             (256, 160, None, 0.0, 64), (2, 300, [300, 200], 0.0, 128),
                                             (256, 160, None, 0.0, 128), (2, 300, [300, 260], 1e4, 128)],
                         ids=["splits", "rope", "one-chunk", "h128-splits", "h128-one-chunk", "h128-rope"])
def test_mla_decode_score_growth_beyond_reference(B, T, ctx, rope, Nh):
    """Scores that grow far past the first tile's max (the decoupled k^R dims of later tokens
    scaled by 200, so V = c^KV stays of order one): such heads leave the fast path's fixed
    reference max and are recomputed exactly; the result still matches the oracle."""
    ctx = np.asarray(ctx if ctx is not None else np.full(B, T), np.int32)
    q = synth.normal(497, 0, (B, Nh, 576), "bf16")
    kf = synth.as_f32(synth.normal(497, 1, (B, T, 1, 576), "bf16"), "bf16").copy()
    kf[:, 40:, :, 512:] *= 200.0
    kc = synth.f32_to_bf16_bits(kf)
    scale = 1.0 / math.sqrt(192)
    # the inputs do leave the fast path's range: some head's later score exceeds its first-tile max
    # by more than 2^64 in the exponent (scale * log2(e) units), checked here without rotation
    qf = synth.as_f32(q, "bf16").astype(np.float64)
    kd = synth.as_f32(kc, "bf16").astype(np.float64)[:, :, 0]
    sl = np.einsum("bhd,btd->bht", qf, kd) * scale * math.log2(math.e)
    assert np.any(sl[:, :, 40:].max(axis=2) > sl[:, :, :32].max(axis=2) + 64)
    got = _gpu_decode(q, kc, None, ctx, scale=scale, rope=rope, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=scale, mla=True, rope=rope)
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("mla,B,Nh", [(False, 3, 8), (False, 600, 8), (False, 3, 16), (False, 600, 32), (True, 3, 64),
                                     (True, 256, 64), (True, 3, 32), (True, 256, 32), (True, 3, 128), (True, 256, 128)],
                         ids=["gqa-split", "gqa-one-chunk", "gqa4-split", "gqa4-one-chunk", "mla64-split",
                              "mla64-one-chunk", "mla32-split", "mla32-one-chunk", "mla128-split", "mla128-one-chunk"])
def test_decode_empty_context_gives_zero_row(mla, B, Nh):
    """A context of 0 keys (a precondition violation the kernels clamp) gives an all-zero output row,
    whether or not the call splits the context (single chunk: no merge follows); the other rows are
    unaffected."""
    T = 96
    ctx = np.full(B, 70, np.int32)
    ctx[0] = 0
    ctx[B // 2] = 0
    wid = 530 + B + Nh
    if mla:
        q = synth.normal(wid, 0, (B, Nh, 576), "bf16")
        kc = synth.normal(wid, 1, (B, T, 1, 576), "bf16")
        vc, kw = None, dict(scale=1.0 / math.sqrt(192), mla=True)
    else:
        Nkv = Nh // 4  # 2, 4 or 8 KV heads of 4 query heads each
        q = synth.normal(wid, 0, (B, Nh, 128), "bf16")
        kc = synth.normal(wid, 1, (B, T, Nkv, 128), "bf16")
        vc, kw = synth.normal(wid, 2, (B, T, Nkv, 128), "bf16"), {}
    got = _gpu_decode(q, kc, vc, ctx, **kw)
    empty = ctx == 0
    assert np.all(got[empty] == 0.0)
    keep = np.flatnonzero(~empty)[:4]
    want = _oracle_decode(q[keep], kc[keep], None if vc is None else vc[keep], ctx[keep], **kw)
    assert max_abs(got[keep], want) <= BF16_TOL


@pytest.mark.parametrize("mla,mla_heads", [(False, 0), (True, 64), (True, 128)], ids=["gqa", "mla64", "mla128"])
def test_decode_padded_cache_rows(mla, mla_heads):
    """Cache rows with a pitch larger than the head dim (the binding passes the stride as the row
    pitch); the padding holds NaN, so reading it would show in the output."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, T = 3, 200
    ctx = np.array([200, 37, 129], np.int32)
    Nh, Nkv, D, pitch = (mla_heads, 1, 576, 640) if mla else (16, 4, 128, 136)
    q = synth.normal(540 + D, 0, (B, Nh, D), "bf16")
    kc = synth.normal(540 + D, 1, (B, T, Nkv, D), "bf16")
    vc = None if mla else synth.normal(540 + D, 2, (B, T, Nkv, D), "bf16")

    def padded(x):
        buf = torch.full((B, T, Nkv, pitch), float("nan"), dtype=torch.bfloat16, device="cuda")
        buf[..., :D] = to_dev(x, "bf16")
        return buf

    kpad = padded(kc)
    vd = kpad[..., :512] if mla else padded(vc)[..., :D]
    scale = 1.0 / math.sqrt(192) if mla else None
    out = attn.decode(to_dev(q, "bf16"), kpad[..., :D], vd, torch.as_tensor(ctx, device="cuda"), scale=scale)
    got = out.float().cpu().numpy()
    want = _oracle_decode(q, kc, vc, ctx, scale=scale, mla=mla)
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= BF16_TOL


def test_mla_decode_never_reads_beyond_context():
    B, Nh, T = 3, 128, 300
    ctx = np.array([7, 150, 300], np.int32)
    q = synth.normal(495, 0, (B, Nh, 576), "bf16")
    kc = synth.normal(495, 1, (B, T, 1, 576), "bf16")
    scale = 1.0 / math.sqrt(192)
    clean = _gpu_decode(q, kc, None, ctx, scale=scale, mla=True)
    kn = kc.copy()
    for b, c in enumerate(ctx):
        kn[b, c:] = 0x7FC0  # bf16 NaN
    dirty = _gpu_decode(q, kn, None, ctx, scale=scale, mla=True)
    assert np.all(np.isfinite(dirty))
    assert np.array_equal(clean, dirty)


def test_llama3_decode_full():
    w = synth.LLAMA3_DECODE
    q, kc, vc, ctx = w.inputs()
    got = _gpu_decode(q, kc, vc, ctx)
    want = _oracle_decode(q, kc, vc, ctx)
    assert got.shape == (64, 32, 128)
    assert max_abs(got, want) <= BF16_TOL


def test_mla_decode_full():
    w = synth.MLA_DECODE
    q, kc, _, ctx = w.inputs()
    got = _gpu_decode(q, kc, None, ctx, scale=w.scale, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=w.scale, mla=True)
    assert got.shape == (32, 128, 512)
    assert max_abs(got, want) <= BF16_TOL


def test_mla_decode_full_rope():
    """The full MLA-absorbed decode with the decoupled q^R rotated in-kernel at position ctx-1."""
    w = synth.MLA_DECODE
    q, kc, _, ctx = w.inputs()
    got = _gpu_decode(q, kc, None, ctx, scale=w.scale, rope=1e4, mla=True)
    want = _oracle_decode(q, kc, None, ctx, scale=w.scale, rope=1e4, mla=True)
    assert max_abs(got, want) <= BF16_TOL


def test_prefill_equals_token_by_token_decode():
    """With and without the KV cache the outputs agree ("Transformer 与 LLM" slide 02): prefill
    with RoPE versus decoding every position against a cache of rotated keys."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, S, Nh, Nkv, D, th = 2, 96, 8, 2, 128, 5e5
    q = to_dev(synth.normal(470, 0, (B, S, Nh, D), "bf16"), "bf16")
    k = to_dev(synth.normal(470, 1, (B, S, Nkv, D), "bf16"), "bf16")
    v = to_dev(synth.normal(470, 2, (B, S, Nkv, D), "bf16"), "bf16")
    full = attn.prefill(q, k, v, rope_theta=th).float()
    kcache = attn.rope_apply_(k.clone(), theta=th)
    worst = 0.0
    for t in range(S):
        ctx = torch.full((B,), t + 1, dtype=torch.int32, device="cuda")
        dec = attn.decode(q[:, t].contiguous(), kcache, v, ctx, rope_theta=th).float()
        worst = max(worst, float((dec - full[:, t]).abs().max()))
    assert worst <= BF16_TOL
