"""KV-cache append (RoPE fused) and prefill against the cache (chunked prefill) on the GPU.

Parity against the oracle (fp64, tolerance BF16_TOL): the appended rows against the oracle's
RoPE at absolute positions; a chunk after a cached prefix against oracle.prefill_chunk.
Consistency inside the library: prefilling a sequence chunk by chunk through the cache gives
bit-for-bit the rows of the single whole-sequence prefill (same rotated keys, same 32-key
blocks in the same order).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import BF16_TOL, max_abs, to_dev, values

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bits(t):
    return t.view(_torch().int16).cpu().numpy()


def _empty_cache(B, T, Nkv, D, ld=None, fill=0x3F80):
    """bf16 cache [B, T, Nkv, ld] filled with a sentinel (1.0), returned as its [..., :D] view."""
    torch = _torch()
    ld = ld or D
    c = torch.full((B, T, Nkv, ld), fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return c[..., :D], c


@pytest.mark.parametrize("D,interleaved,rope,rdims", [(128, False, 5e5, 0), (64, True, 1e4, 0), (128, False, 0.0, 0),
                                                      (128, False, 1e4, 64), (64, True, 5e5, 32)])
def test_kv_append_rotates_and_places(D, interleaved, rope, rdims):
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, S, Nkv, T = 2, 37, 2, 100
    start = np.array([0, 50], np.int32)
    kn = synth.normal(800 + D, 0, (B, S, Nkv, D), "bf16")
    vn = synth.normal(800 + D, 1, (B, S, Nkv, D), "bf16")
    kc, kc_full = _empty_cache(B, T, Nkv, D, ld=D + 8)
    vc, _ = _empty_cache(B, T, Nkv, D)
    attn.kv_append(to_dev(kn, "bf16"), to_dev(vn, "bf16"), kc, vc, torch.as_tensor(start, device="cuda"),
                   rope_theta=rope, rope_dims=rdims, interleaved=interleaved)
    kh = kc.float().cpu().numpy()
    vh = _bits(vc)
    for b in range(B):
        rows = slice(start[b], start[b] + S)
        want = values(kn[b:b + 1], "bf16")
        if rope > 0:
            want = oracle.rope_rotate(want, start[b] + np.arange(S), rope, interleaved=interleaved,
                                      rot_dims=rdims or None)
        assert max_abs(kh[b, rows], want[0]) <= BF16_TOL
        if rope == 0:
            assert np.array_equal(_bits(kc[b, rows].contiguous()), kn[b].view(np.int16))
        assert np.array_equal(vh[b, rows], vn[b].view(np.int16))
        others = np.ones(T, bool)
        others[rows] = False
        assert np.all(kh[b, others] == 1.0) and np.all(vh[b, others] == 0x3F80)
    # the row padding beyond D is never written
    assert np.all(kc_full[..., D:].float().cpu().numpy() == 1.0)


@pytest.mark.parametrize("D,interleaved,rdims", [(128, False, 0), (64, True, 0), (128, False, 36)])
def test_kv_append_scalar_path_gives_the_vector_paths_bits(D, interleaved, rdims):
    """A row pitch of D + 2 elements rules out 16-byte accesses, so the append takes its element-wise
    path; its rows must carry the same bits as the 16-byte path's (which the test above pins to the
    oracle). rdims = 36 (half = 18) also makes the 16-byte path fetch partners one by one."""
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, S, Nkv, T = 2, 21, 2, 64
    start = torch.as_tensor(np.array([3, 40], np.int32), device="cuda")
    kn = to_dev(synth.normal(820 + D, 0, (B, S, Nkv, D), "bf16"), "bf16")
    vn = to_dev(synth.normal(820 + D, 1, (B, S, Nkv, D), "bf16"), "bf16")
    caches = []
    for ld in (D, D + 2):
        kc, _ = _empty_cache(B, T, Nkv, D, ld=ld)
        vc, _ = _empty_cache(B, T, Nkv, D, ld=ld)
        attn.kv_append(kn, vn, kc, vc, start, rope_theta=1e4, rope_dims=rdims, interleaved=interleaved)
        caches.append((_bits(kc.contiguous()), _bits(vc.contiguous())))
    assert np.array_equal(caches[0][0], caches[1][0])
    assert np.array_equal(caches[0][1], caches[1][1])


CHUNK_CASES = [
    # B, S, Nh, Nkv, D, T, starts, rope, causal
    (2, 33, 8, 2, 128, 128, [0, 45], 5e5, True),
    (2, 70, 4, 4, 64, 200, [130, 3], 0.0, True),
    (3, 1, 8, 1, 128, 64, [0, 17, 63], 1e4, True),
    (1, 40, 4, 2, 128, 96, [56], 0.0, False),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "S%dH%dK%dD%d" % c[1:5])
def test_prefill_cached_matches_oracle(case):
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, S, Nh, Nkv, D, T, starts, rope, causal = case
    wid = 820 + S
    starts = np.asarray(starts, np.int32)
    k_all = synth.normal(wid, 1, (B, T, Nkv, D), "bf16")
    v_all = synth.normal(wid, 2, (B, T, Nkv, D), "bf16")
    q = synth.normal(wid, 0, (B, S, Nh, D), "bf16")
    kc, _ = _empty_cache(B, T, Nkv, D)
    vc, _ = _empty_cache(B, T, Nkv, D)
    # fill each sequence's first start+S rows through the append kernel (rotated keys)
    n_max = int((starts + S).max())
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    attn.kv_append(to_dev(k_all[:, :n_max], "bf16"), to_dev(v_all[:, :n_max], "bf16"), kc, vc, zeros,
                   rope_theta=rope)
    got = attn.prefill_cached(to_dev(q, "bf16"), kc, vc, torch.as_tensor(starts, device="cuda"),
                              rope_theta=rope, causal=causal).float().cpu().numpy()
    want = oracle.prefill_chunk(values(q, "bf16"), values(k_all, "bf16"), values(v_all, "bf16"), starts,
                                causal=causal, rope_theta=rope)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("chunks,rope", [([64, 100, 93], 5e5), ([1, 31, 32, 33, 160], 0.0)])
def test_chunked_prefill_is_bitwise_the_full_prefill(chunks, rope):
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, Nh, Nkv, D = 2, 8, 2, 128
    T = sum(chunks)
    q = to_dev(synth.normal(840, 0, (B, T, Nh, D), "bf16"), "bf16")
    k = to_dev(synth.normal(840, 1, (B, T, Nkv, D), "bf16"), "bf16")
    v = to_dev(synth.normal(840, 2, (B, T, Nkv, D), "bf16"), "bf16")
    full = attn.prefill(q, k, v, rope_theta=rope)
    kc, _ = _empty_cache(B, T, Nkv, D)
    vc, _ = _empty_cache(B, T, Nkv, D)
    outs, s0 = [], 0
    for n in chunks:
        st = torch.full((B,), s0, dtype=torch.int32, device="cuda")
        attn.kv_append(k[:, s0:s0 + n].contiguous(), v[:, s0:s0 + n].contiguous(), kc, vc, st, rope_theta=rope)
        outs.append(attn.prefill_cached(q[:, s0:s0 + n].contiguous(), kc, vc, st, rope_theta=rope))
        s0 += n
    assert np.array_equal(_bits(torch.cat(outs, dim=1)), _bits(full))


WINDOW_CASES = [
    # B, S, Nh, Nkv, D, T, starts, rope, window, sinks
    (2, 200, 8, 2, 128, 256, [0, 56], 5e5, 64, 4),
    (1, 96, 4, 4, 64, 300, [204], 0.0, 100, 0),
    (2, 130, 4, 1, 128, 130, [0, 0], 1e4, 33, 40),
    (1, 64, 4, 2, 128, 64, [0], 0.0, 1, 0),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "S%dD%dW%dK%d" % (c[1], c[4], c[8], c[9]))
def test_sliding_window_with_sinks_matches_oracle(case):
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, S, Nh, Nkv, D, T, starts, rope, window, sinks = case
    wid = 860 + S + window
    starts = np.asarray(starts, np.int32)
    k_all = synth.normal(wid, 1, (B, T, Nkv, D), "bf16")
    v_all = synth.normal(wid, 2, (B, T, Nkv, D), "bf16")
    q = synth.normal(wid, 0, (B, S, Nh, D), "bf16")
    kc, _ = _empty_cache(B, T, Nkv, D)
    vc, _ = _empty_cache(B, T, Nkv, D)
    n_max = int((starts + S).max())
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    attn.kv_append(to_dev(k_all[:, :n_max], "bf16"), to_dev(v_all[:, :n_max], "bf16"), kc, vc, zeros,
                   rope_theta=rope)
    got = attn.prefill_cached(to_dev(q, "bf16"), kc, vc, torch.as_tensor(starts, device="cuda"),
                              rope_theta=rope, window=window, sinks=sinks).float().cpu().numpy()
    want = oracle.prefill_chunk(values(q, "bf16"), values(k_all, "bf16"), values(v_all, "bf16"), starts,
                                rope_theta=rope, window=window, sinks=sinks)
    assert max_abs(got, want) <= BF16_TOL


def test_sliding_window_score_growth_beyond_reference():
    """Window + sinks with keys whose scores lie far above those of each query's first visible
    block (keys 100.. scaled after bf16 widening): the exact path of the softmax keeps the result
    equal to the oracle's."""
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    B, S, Nh, Nkv, D, T, window, sinks = 1, 256, 4, 2, 128, 256, 64, 4
    k_all = synth.as_f32(synth.normal(880, 1, (B, T, Nkv, D), "bf16"), "bf16").copy()
    k_all[:, 100:] *= 20.0
    k_all = synth.f32_to_bf16_bits(k_all)
    v_all = synth.normal(880, 2, (B, T, Nkv, D), "bf16")
    q = synth.normal(880, 0, (B, S, Nh, D), "bf16")
    kc, _ = _empty_cache(B, T, Nkv, D)
    vc, _ = _empty_cache(B, T, Nkv, D)
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    attn.kv_append(to_dev(k_all, "bf16"), to_dev(v_all, "bf16"), kc, vc, zeros)
    got = attn.prefill_cached(to_dev(q, "bf16"), kc, vc, zeros, window=window, sinks=sinks).float().cpu().numpy()
    want = oracle.prefill_chunk(values(q, "bf16"), values(k_all, "bf16"), values(v_all, "bf16"), np.zeros(B, np.int32),
                                window=window, sinks=sinks)
    assert np.all(np.isfinite(got))
    assert max_abs(got, want) <= BF16_TOL


ROPE_CASES = [
    # D, rope_dims, interleaved, theta
    (128, 64, False, 1e4),
    (128, 128, True, 5e5),
    (64, 32, True, 1e4),
    (128, 32, False, 5e5),
    (128, 96, False, 1e4),  # three register pairs of the half-split q rotation
    (128, 96, True, 1e4),
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "D%dR%d%s" % (c[0], c[1], "i" if c[2] else "h"))
def test_prefill_cached_rope_variants_match_oracle(case):
    """Adjacent-pair and partial rotary RoPE in the fused path: the append rotates K, the prefill
    rotates q in registers, both over the same span and pairing."""
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    D, rdims, inter, theta = case
    B, S, Nh, Nkv, T = 2, 48, 8, 2, 128
    starts = np.array([0, 70], np.int32)
    wid = 880 + D + rdims
    k_all = synth.normal(wid, 1, (B, T, Nkv, D), "bf16")
    v_all = synth.normal(wid, 2, (B, T, Nkv, D), "bf16")
    q = synth.normal(wid, 0, (B, S, Nh, D), "bf16")
    kc, _ = _empty_cache(B, T, Nkv, D)
    vc, _ = _empty_cache(B, T, Nkv, D)
    n_max = int((starts + S).max())
    zeros = torch.zeros(B, dtype=torch.int32, device="cuda")
    attn.kv_append(to_dev(k_all[:, :n_max], "bf16"), to_dev(v_all[:, :n_max], "bf16"), kc, vc, zeros,
                   rope_theta=theta, rope_dims=rdims, interleaved=inter)
    got = attn.prefill_cached(to_dev(q, "bf16"), kc, vc, torch.as_tensor(starts, device="cuda"), rope_theta=theta,
                              rope_dims=rdims, rope_interleaved=inter).float().cpu().numpy()
    want = oracle.prefill_chunk(values(q, "bf16"), values(k_all, "bf16"), values(v_all, "bf16"), starts,
                                rope_theta=theta, rope_interleaved=inter, rope_dims=rdims)
    assert max_abs(got, want) <= BF16_TOL


def _llama3_full_size_rows(window, sinks):
    """The Llama-3-8B-shaped prefill (B=4, S=8192, 32/8 heads of 128, RoPE 5e5) run the way the
    benchmark's widened rows run it: the cache filled by four 2048-token appends (RoPE fused), then
    either each chunk's queries against the cache (window 0) or all 8192 queries at once with a
    sliding window. Returns (output rows [4, R, 32, 128], the oracle's, the rows)."""
    import causal_head_attention_gqa_amd as attn
    torch = _torch()
    w = synth.LLAMA3_PREFILL
    B, S, Nh, Nkv, D, theta, C = w.B, w.S, w.Nh, w.Nkv, w.Dh, w.rope_theta, 2048
    q, k, v = w.inputs()
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kcache = torch.empty((B, S, Nkv, D), dtype=torch.bfloat16, device="cuda")
    vcache = torch.empty_like(kcache)
    out = torch.empty_like(qd)
    for c in range(0, S, C):
        start = torch.full((B,), c, dtype=torch.int32, device="cuda")
        attn.kv_append(kd[:, c:c + C].contiguous(), vd[:, c:c + C].contiguous(), kcache, vcache, start,
                       rope_theta=theta)
        if window == 0:
            out[:, c:c + C] = attn.prefill_cached(qd[:, c:c + C].contiguous(), kcache, vcache, start, rope_theta=theta)
    if window > 0:
        zero = torch.zeros((B,), dtype=torch.int32, device="cuda")
        attn.prefill_cached(qd, kcache, vcache, zero, rope_theta=theta, window=window, sinks=sinks, out=out)
    # chunk and tile edges, window edges, the last row, and rows drawn at random
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 2047, 2048, 2049, 4095, 4096, 4099, 4100, 6143, 6144, 8191],
                                     np.random.default_rng(11).integers(0, S, 26)]))
    got = out[:, torch.as_tensor(rows, device=out.device)].float().cpu().numpy()
    # oracle: each row is a one-token chunk at its position; q and k rotated once by the oracle's RoPE
    # (the same rotation prefill_chunk applies, so rope_theta=0 there)
    kv_, vv = values(k, "bf16"), values(v, "bf16")
    want = np.empty(got.shape)
    for b in range(B):
        kr = oracle.rope_rotate(kv_[b:b + 1], np.arange(S), theta)
        qr = oracle.rope_rotate(values(q[b:b + 1, rows], "bf16"), rows, theta)
        for i, r in enumerate(rows):
            want[b, i] = oracle.prefill_chunk(qr[:, i:i + 1], kr[:, :r + 1], vv[b:b + 1, :r + 1], [int(r)],
                                              window=window, sinks=sinks)[0, 0]
    return got, want, rows


def test_llama3_chunked_prefill_full_size_sampled_rows():
    """Four 2048-token chunks with fused RoPE append, at the Llama-3-8B size the benchmark times."""
    got, want, rows = _llama3_full_size_rows(0, 0)
    assert max_abs(got, want) <= BF16_TOL


def test_llama3_sliding_window_full_size_sampled_rows():
    """Window 4096 + 4 sinks over the whole 8192-token sequence, the size the benchmark times."""
    got, want, rows = _llama3_full_size_rows(4096, 4)
    assert max_abs(got, want) <= BF16_TOL


@pytest.mark.parametrize("window,sinks", [(0, 0), (300, 4)], ids=["causal", "window"])
def test_prefill_cached_work_lists_give_the_static_order_bits(window, sinks):
    """Chunked prefill against a cache: the optional work-list counters at the end of the workspace
    only change which work-group takes a q-tile; the output equals, bit for bit, that of a call
    whose workspace stops short of them (16 (sequence, head group) pairs: one list per XCD)."""
    import causal_head_attention_gqa_amd as attn
    torch = __import__("torch")
    B, S, Nh, Nkv, D, T, theta = 2, 512, 32, 8, 128, 1536, 5e5
    wid = 940 + window
    kc = to_dev(synth.normal(wid, 1, (B, T, Nkv, D), "bf16"), "bf16")
    vc = to_dev(synth.normal(wid, 2, (B, T, Nkv, D), "bf16"), "bf16")
    q = to_dev(synth.normal(wid, 0, (B, S, Nh, D), "bf16"), "bf16")
    start = torch.tensor([T - S, 400], dtype=torch.int32, device="cuda")
    full = attn.prefill_cached_workspace_bytes(T, D, theta)
    buf = torch.full((full + 4096,), 0xA5, dtype=torch.uint8, device="cuda")  # canary past the figure
    kw = dict(rope_theta=theta, window=window, sinks=sinks)
    listed = attn.prefill_cached(q, kc, vc, start, workspace=buf[:full], **kw)
    torch.cuda.synchronize()
    assert bool((buf[full:] == 0xA5).all())
    static = attn.prefill_cached(q, kc, vc, start, workspace=buf[:full - 512], **kw)
    assert torch.isfinite(listed.float()).all()
    assert torch.equal(listed, static)
