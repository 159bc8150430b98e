"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it follows. A plausible mistake in the oracle (a dropped scale, a
wrong sign in the rotation, the wrong pairing or frequency index, a transposed product, a
mask on the wrong side of the diagonal, the wrong GQA head mapping, V taken from the wrong part
of the MLA row) fails at least one of them.
"""
import math

import numpy as np
import pytest

import oracle
from causal_head_attention_gqa_amd import accounting


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------------------------ mask ----
@pytest.mark.parametrize("S,name", [(4, "causal_mask_s4.txt"), (5, "causal_mask_s5.txt")])
def test_mask_matches_printed_matrix(S, name, golden):
    """"2.7 Transformer Decoder Block完整解析" §3.2 and §3.3 print the 5x5 and 4x4 masks."""
    printed = np.array([[float(x) for x in row] for row in golden(name)])
    m = oracle.causal_mask(np.arange(S), S)
    assert m.shape == printed.shape
    assert np.array_equal(m, printed)


def test_visibility_matches_printed_table(golden):
    """§3.2 of the same page prints which keys each query sees (lower triangle)."""
    printed = np.array([[int(x) for x in row] for row in golden("causal_visibility_s5.txt")])
    vis = (oracle.causal_mask(np.arange(5), 5) == 0).astype(int)
    assert np.array_equal(vis, printed)


# ------------------------------------------------------------- worked single-head example ----
def test_single_head_d4_t3_constructed_case(golden):
    """Slide 01 of "Transformer 与 LLM" prints t2's weights (0.27, 0.27, 0.45) for d=4, T=3.

    The slide's inputs are not in the text. This constructed case has d=4, T=3, scale 1/sqrt(4):
    q_2 = e_0, k_0 = k_1 = 0, k_2 = e_0, v_j = e_j. Its exact weights for t2 are
    (1, 1, sqrt(e)) / (2 + sqrt(e)), which round to the printed values; rows 0 and 1 are
    (1, 0, 0) and (1/2, 1/2, 0).
    """
    rows = golden("head_d4_t3_weights.txt")
    printed = [float(x) for x in rows[0][1:]]
    decimals = int(rows[1][1])
    q = np.zeros((1, 3, 1, 4))
    q[0, :, 0, 0] = 1.0
    k = np.zeros((1, 3, 1, 4))
    k[0, 2, 0, 0] = 1.0
    v = np.zeros((1, 3, 1, 4))
    for j in range(3):
        v[0, j, 0, j] = 1.0
    out = oracle.prefill(q, k, v, causal=True)  # scale defaults to 1/sqrt(d)
    se = math.sqrt(math.e)
    exact_t2 = np.array([1.0, 1.0, se, 0.0]) / (2.0 + se)
    np.testing.assert_allclose(out[0, 2, 0], exact_t2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0, 0], [1, 0, 0, 0], rtol=0, atol=0)
    np.testing.assert_allclose(out[0, 1, 0], [0.5, 0.5, 0, 0], rtol=0, atol=1e-15)
    assert [round(x, decimals) for x in out[0, 2, 0, :3]] == printed


# ------------------------------------------------------------------------- softmax / mask ----
def test_rows_sum_to_one_and_masked_weights_are_zero():
    """"Transformer 架构完全深度解析" §五 step 4: each row of A sums to 1; masked entries get 0."""
    rng = np.random.default_rng(0)
    q, k = _rand(rng, 37, 16), _rand(rng, 37, 16)
    a = oracle.attention_weights(q, k, 0.25, oracle.causal_mask(np.arange(37), 37))
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(a[np.triu_indices(37, 1)] == 0.0)
    assert np.all(a[np.tril_indices(37)] > 0.0)


def test_softmax_closed_form_two_entries():
    """softmax(x, x + t) = (1, e^t) / (1 + e^t) (textbook two-entry softmax)."""
    for t in (-3.0, 0.0, 0.7, 20.0):
        p = oracle.softmax_rows(np.array([[1.5, 1.5 + t]]))
        np.testing.assert_allclose(p[0], [1 / (1 + math.exp(t)), math.exp(t) / (1 + math.exp(t))],
                                   rtol=1e-14, atol=1e-300)


def test_softmax_survives_large_scores():
    """The softmax of "Transformer 架构快速入门" §4.4 is exp(s_j) / sum_k exp(s_k) for any scores; it
    is invariant to a common shift, so two keys whose scores differ by ln 2 get weights 2/3 and
    1/3 whether the scores sit near +1000 or -1000 (where exp alone overflows or underflows)."""
    for base in (1000.0, -1000.0, 0.0):
        s = np.array([[base, base - math.log(2.0)]])
        np.testing.assert_allclose(oracle.softmax_rows(s), [[2.0 / 3.0, 1.0 / 3.0]], rtol=1e-12)
    q = np.array([[40.0]])
    k = np.array([[50.0], [50.0 - math.log(2.0) / 40.0]])
    np.testing.assert_allclose(oracle.attention_weights(q, k, 1.0), [[2.0 / 3.0, 1.0 / 3.0]], rtol=1e-9)


def test_scale_divides_by_head_dim():
    """"Transformer 架构快速入门" §4.3: scores are divided by sqrt(D_h), per head dim.

    Two keys whose raw dot products with q differ by D: weight ratio must be exp(D / sqrt(D))."""
    D = 64
    q = np.zeros((1, D)); q[0, :] = 1.0
    k = np.zeros((2, D)); k[1, :] = 1.0
    a = oracle.attention_weights(q, k, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(a[0, 1] / a[0, 0], math.exp(D / math.sqrt(D)), rtol=1e-12)


def test_row0_attends_only_to_itself():
    """§3.2 of the decoder-block page: t0 only sees itself, so out_0 = v_0 exactly."""
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 2, 9, 4, 8), _rand(rng, 2, 9, 2, 8), _rand(rng, 2, 9, 2, 8)
    out = oracle.prefill(q, k, v, causal=True, rope_theta=1e4)
    for h in range(4):
        assert np.array_equal(out[:, 0, h, :], v[:, 0, h // 2, :])


def test_future_rows_do_not_change_past_outputs():
    """The causal constraint of the decoder-block page §3.1: edits to keys/values after t leave
    outputs up to t unchanged, and a prefix's prefill equals the prefix of the full prefill."""
    rng = np.random.default_rng(2)
    q, k, v = _rand(rng, 1, 12, 2, 8), _rand(rng, 1, 12, 2, 8), _rand(rng, 1, 12, 2, 8)
    base = oracle.prefill(q, k, v, rope_theta=500.0)
    k2, v2 = k.copy(), v.copy()
    k2[:, 7:] += 5.0
    v2[:, 7:] -= 3.0
    pert = oracle.prefill(q, k2, v2, rope_theta=500.0)
    assert np.array_equal(base[:, :7], pert[:, :7])
    assert not np.allclose(base[:, 7:], pert[:, 7:])
    prefix = oracle.prefill(q[:, :5], k[:, :5], v[:, :5], rope_theta=500.0)
    np.testing.assert_allclose(prefix, base[:, :5], rtol=0, atol=1e-14)


def test_equal_keys_give_prefix_means():
    """With identical keys every visible score is equal, so output i is the mean of the visible
    values ("Transformer 架构快速入门" §4.5 weighted sum with uniform weights)."""
    rng = np.random.default_rng(3)
    S, D = 10, 6
    q = _rand(rng, 1, S, 1, D)
    k = np.broadcast_to(_rand(rng, 1, 1, 1, D), (1, S, 1, D)).copy()
    v = _rand(rng, 1, S, 1, D)
    out = oracle.prefill(q, k, v, causal=True)
    want = np.cumsum(v[0, :, 0, :], axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(out[0, :, 0, :], want, rtol=0, atol=1e-14)
    out_full = oracle.prefill(q, k, v, causal=False)
    np.testing.assert_allclose(out_full[0, :, 0, :], np.broadcast_to(v[0, :, 0, :].mean(0), (S, D)),
                               rtol=0, atol=1e-14)


def test_permutation_equivariance_without_mask_or_position():
    """"Transformer 架构快速入门" §7 and slide 01 of "Transformer 与 LLM": with no mask and no
    position information, permuting the tokens permutes the outputs."""
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 11, 4, 8), _rand(rng, 2, 11, 2, 8), _rand(rng, 2, 11, 2, 8)
    perm = rng.permutation(11)
    out = oracle.prefill(q, k, v, causal=False)
    out_p = oracle.prefill(q[:, perm], k[:, perm], v[:, perm], causal=False)
    np.testing.assert_allclose(out_p, out[:, perm], rtol=0, atol=1e-13)
    # and the causal mask breaks it (the mask carries order)
    assert not np.allclose(oracle.prefill(q[:, perm], k[:, perm], v[:, perm], causal=True),
                           oracle.prefill(q, k, v, causal=True)[:, perm])


def test_gqa_equals_mha_with_repeated_kv():
    """"Transformer 架构快速入门" §6.3: query heads 1-4 share KV head 1, ..., 29-32 share KV head 8.
    GQA must equal MHA whose K/V heads are repeated G times in that order."""
    rng = np.random.default_rng(5)
    Nh, Nkv = 8, 2
    q, k, v = _rand(rng, 1, 13, Nh, 8), _rand(rng, 1, 13, Nkv, 8), _rand(rng, 1, 13, Nkv, 8)
    gqa = oracle.prefill(q, k, v, rope_theta=1e4)
    mha = oracle.prefill(q, np.repeat(k, Nh // Nkv, axis=2), np.repeat(v, Nh // Nkv, axis=2), rope_theta=1e4)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-14)
    assert [oracle.kv_head_of(h, 32, 8) for h in (0, 3, 4, 31)] == [0, 0, 1, 7]


# -------------------------------------------------------------------------------------- RoPE --
def test_rope_two_dims_is_plane_rotation():
    """D=2: theta_0 = 1, so position m rotates (1,0) to (cos m, sin m) and (0,1) to (-sin m, cos m)
    ("Transformer 架构快速入门" §8.3 rotation matrix R(alpha))."""
    m = np.array([0, 1, 5, 1000])
    x = np.zeros((1, 4, 2, 2)); x[..., 0, 0] = 1.0; x[..., 1, 1] = 1.0
    r = oracle.rope_rotate(x, m, 777.0)
    np.testing.assert_allclose(r[0, :, 0], np.stack([np.cos(m), np.sin(m)], 1), atol=1e-15)
    np.testing.assert_allclose(r[0, :, 1], np.stack([-np.sin(m), np.cos(m)], 1), atol=1e-15)


def test_rope_pair_index_and_frequency():
    """D=4 half-split pairs (0,2) and (1,3) ("2.7 ..." §4 apply_rope). Pair 1 has frequency
    base^(-2/4) ("Transformer 架构快速入门" §8.2, 0-based i)."""
    base, m = 10000.0, 7
    x = np.zeros((1, 1, 1, 4)); x[..., 1] = 1.0
    r = oracle.rope_rotate(x, [m], base)[0, 0, 0]
    a = m * base ** -0.5
    np.testing.assert_allclose(r, [0.0, math.cos(a), 0.0, math.sin(a)], atol=1e-15)
    xi = np.zeros((1, 1, 1, 4)); xi[..., 2] = 1.0   # interleaved: pair (2, 3) is pair 1
    ri = oracle.rope_rotate(xi, [m], base, interleaved=True)[0, 0, 0]
    np.testing.assert_allclose(ri, [0.0, 0.0, math.cos(a), math.sin(a)], atol=1e-15)


def test_rope_position_zero_is_identity_and_norm_is_kept():
    rng = np.random.default_rng(6)
    x = _rand(rng, 2, 9, 3, 16)
    r = oracle.rope_rotate(x, np.arange(9), 1e4)
    assert np.array_equal(r[:, 0], x[:, 0])
    pair_norm = lambda t: t[..., :8] ** 2 + t[..., 8:] ** 2  # noqa: E731
    np.testing.assert_allclose(pair_norm(r), pair_norm(x), rtol=1e-13)


def test_rope_relative_position_identity():
    """"Transformer 架构快速入门" §8.4: R(m)^T R(n) = R(n - m), so <R_m q, R_n k> depends on n - m."""
    rng = np.random.default_rng(7)
    q, k = _rand(rng, 1, 1, 1, 32), _rand(rng, 1, 1, 1, 32)
    def dot(m, n):
        return float(np.sum(oracle.rope_rotate(q, [m], 5e5) * oracle.rope_rotate(k, [n], 5e5)))
    for m, n, d in ((3, 8, 10), (0, 0, 99), (100, 40, 7)):
        assert dot(m, n) == pytest.approx(dot(m + d, n + d), rel=1e-10, abs=1e-10)
    assert dot(3, 8) != pytest.approx(dot(3, 9), rel=1e-6)


def test_rope_pairings_differ_by_fixed_permutation():
    """"Transformer 架构快速入门" §8.1: adjacent and half-split pairing are the same rotation on a
    reordered vector: interleaved(x) = P^-1 halfsplit(P x) with P = evens then odds."""
    rng = np.random.default_rng(8)
    D = 16
    x = _rand(rng, 2, 5, 3, D)
    P = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])
    inv = np.argsort(P)
    hs = oracle.rope_rotate(x[..., P], np.arange(5), 1e4)
    np.testing.assert_allclose(oracle.rope_rotate(x, np.arange(5), 1e4, interleaved=True), hs[..., inv],
                               rtol=0, atol=1e-15)


def test_rope_wavelength_count_matches_printed(golden):
    """Slide 07 of "Transformer 与 LLM": 14 pairs of 64 do not finish a turn within 8K at base 1e4.
    A 1-based frequency index would give 15."""
    D, base, ctx, n = (float(x) for x in golden("rope_wavelength.txt")[0])
    wavelength = 2 * math.pi / oracle.rope_inv_freq(int(D), base)
    assert int(np.sum(wavelength > ctx)) == int(n)


def test_rope_only_q_and_k():
    """V is not rotated ("2.7 ..." §2, "Transformer 架构快速入门" §8.5): rotating v changes output,
    rotating q and k by the same position shift does not (relative identity at work)."""
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 1, 6, 1, 8), _rand(rng, 1, 6, 1, 8), _rand(rng, 1, 6, 1, 8)
    a = oracle.prefill(q, k, v, rope_theta=1e4)
    qr = oracle.rope_rotate(q, np.arange(6), 1e4)
    kr = oracle.rope_rotate(k, np.arange(6), 1e4)
    b = oracle.prefill(qr, kr, v, rope_theta=0.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------ decode --
def test_decode_equals_prefill_row_by_row():
    """Slide 02 of "Transformer 与 LLM": outputs with and without the KV cache are identical;
    "Transformer 架构完全深度解析" §九: append the new K/V, then attend the new query to the cache."""
    rng = np.random.default_rng(10)
    B, S, Nh, Nkv, D, th = 2, 17, 6, 2, 16, 1e4
    q, k, v = _rand(rng, B, S, Nh, D), _rand(rng, B, S, Nkv, D), _rand(rng, B, S, Nkv, D)
    full = oracle.prefill(q, k, v, rope_theta=th)
    kcache = oracle.rope_rotate(k, np.arange(S), th)
    for t in range(S):
        dec = oracle.decode(q[:, t], kcache, v, np.full(B, t + 1), rope_theta=th)
        np.testing.assert_allclose(dec, full[:, t], rtol=0, atol=1e-13)


def test_decode_ignores_rows_beyond_context():
    rng = np.random.default_rng(11)
    q, kc, vc = _rand(rng, 3, 4, 8), _rand(rng, 3, 20, 2, 8), _rand(rng, 3, 20, 2, 8)
    ctx = np.array([1, 7, 20])
    a = oracle.decode(q, kc, vc, ctx)
    kc2, vc2 = kc.copy(), vc.copy()
    for b, c in enumerate(ctx):
        kc2[b, c:] = np.nan
        vc2[b, c:] = np.nan
    assert np.array_equal(a, oracle.decode(q, kc2, vc2, ctx))
    # ctx = 1: the only key is the query's own token
    assert np.array_equal(a[0], vc[0, 0, [0, 0, 1, 1]])


def test_mla_absorbed_equals_non_absorbed():
    """Slide 06 of "Transformer 与 LLM": absorbing W_UK into the query and W_UV into the output turns
    MLA decode into MQA with 128 heads sharing one 576-dim row [c^KV ; k^R] (V = c^KV), scale
    1/sqrt(192), and gives the same result as per-head attention over q.[k^C ; k^R] / sqrt(192)."""
    rng = np.random.default_rng(12)
    H, T, dc, dr, dh = 8, 33, 512, 64, 128
    c = _rand(rng, T, dc) * 0.05
    kr = _rand(rng, T, dr)
    qc, qr = _rand(rng, H, dh) * 0.1, _rand(rng, H, dr)
    w_uk, w_uv = _rand(rng, H, dh, dc) * 0.05, _rand(rng, H, dh, dc) * 0.05
    scale = 1.0 / math.sqrt(dh + dr)
    ref = np.stack([
        oracle.head_attention(np.concatenate([qc[h], qr[h]])[None],
                              np.concatenate([c @ w_uk[h].T, kr], axis=1), c @ w_uv[h].T, scale)[0]
        for h in range(H)])
    q_abs = np.concatenate([np.einsum("hd,hdc->hc", qc, w_uk), qr], axis=1)[None]  # [1, H, 576]
    row = np.concatenate([c, kr], axis=1)[None, :, None, :]  # [1, T, 1, 576]
    lat = oracle.decode(q_abs, row, row[..., :dc], np.array([T]), scale=scale)[0]  # [H, 512]
    got = np.einsum("hdc,hc->hd", w_uv, lat)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


# -------------------------------------------------------------------------------- accounting --
def test_kv_bytes_per_token_closed_forms(golden):
    rows = golden("kv_cache_bytes.txt")
    for name, L, nkv, d, b, want in rows[:3]:
        assert accounting.kv_bytes_per_token(int(L), int(nkv), int(d), int(b)) == int(want), name
    name, L, row, b, kib = rows[3]
    assert round(accounting.mla_bytes_per_token(int(L), int(row), int(b)) / 1024, 1) == float(kib)


def test_mla_and_logits_accounting(golden):
    rows = {r[0]: float(r[1]) for r in golden("mla_absorbed_accounting.txt")}
    assert round(accounting.mla_absorbed_intensity()) == rows["absorbed_intensity_flop_per_byte"]
    assert round(accounting.mla_absorbed_flop_ratio(), 1) == rows["absorbed_flop_ratio"]
    assert accounting.logits_bytes(8192, 32, 2) == rows["logits_bytes_8k_32heads_bf16"]


def test_prefill_flop_count():
    """4*Dh FLOPs per unmasked pair; the Llama-3-8B-shaped prefill totals 2,199,291,691,008."""
    assert accounting.prefill_flops(4, 8192, 32, 128, causal=True) == 2_199_291_691_008
    assert accounting.prefill_flops(8, 1024, 12, 64, causal=True) == 12_897_484_800
    assert accounting.prefill_flops(1, 3, 1, 4, causal=False) == 4 * 4 * 9
    # MLA non-absorbed prefill: 2 * (192 + 128) FLOPs per pair; the attention FLOP ratio of the absorbed
    # form ([P4] slide 06: about 3.4x) is the ratio of these per-pair counts
    mla = accounting.prefill_flops(1, 4096, 128, 192, causal=True, Dv=128)
    assert mla == 2 * 320 * 128 * (4096 * 4097 // 2)
    assert round(2 * (576 + 512) / (2 * (192 + 128)), 1) == round(accounting.mla_absorbed_flop_ratio(), 1) == 3.4


# ------------------------------------------------------------------ prefill against a cache --
@pytest.mark.parametrize("rope", [0.0, 1e4])
def test_prefill_chunk_equals_rows_of_the_full_prefill(rope):
    """Chunks after a cached prefix reproduce the matching rows of the whole-sequence prefill
    (absolute positions for the mask and for RoPE): a chunk masked or rotated with local
    positions fails this."""
    rng = np.random.default_rng(21)
    B, T, Nh, Nkv, D = 2, 37, 4, 2, 8
    q, k, v = _rand(rng, B, T, Nh, D), _rand(rng, B, T, Nkv, D), _rand(rng, B, T, Nkv, D)
    full = oracle.prefill(q, k, v, rope_theta=rope)
    for off, S in [(0, 37), (0, 5), (11, 9), (30, 7), (36, 1)]:
        got = oracle.prefill_chunk(q[:, off:off + S], k, v, [off] * B, rope_theta=rope)
        np.testing.assert_allclose(got, full[:, off:off + S], rtol=1e-12, atol=1e-13)


def test_prefill_chunk_single_token_is_decode():
    """A one-token chunk at position p is the decode step with p+1 cached keys."""
    rng = np.random.default_rng(22)
    B, T, Nh, Nkv, D = 3, 20, 4, 1, 8
    q, k, v = _rand(rng, B, 1, Nh, D), _rand(rng, B, T, Nkv, D), _rand(rng, B, T, Nkv, D)
    start = np.array([0, 7, 19])
    got = oracle.prefill_chunk(q, k, v, start, rope_theta=5e5)[:, 0]
    krot = oracle.rope_rotate(k, np.arange(T), 5e5)
    want = oracle.decode(q[:, 0], krot, v, start + 1, rope_theta=5e5)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_prefill_chunk_non_causal_sees_the_whole_prefix():
    """Without the mask every query sees keys 0 .. q_start+S-1: the last chunk of a non-causal
    prefill equals those rows of the full non-causal prefill."""
    rng = np.random.default_rng(23)
    B, T, Nh, Nkv, D = 1, 24, 2, 2, 8
    q, k, v = _rand(rng, B, T, Nh, D), _rand(rng, B, T, Nkv, D), _rand(rng, B, T, Nkv, D)
    full = oracle.prefill(q, k, v, causal=False)
    got = oracle.prefill_chunk(q[:, 16:], k, v, [16], causal=False)
    np.testing.assert_allclose(got, full[:, 16:], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ sliding window + attention sinks --
def test_window_sink_visibility_matches_hand_table(golden):
    """W = 3, one sink, six tokens: the hand-written visibility table of the rule."""
    table = np.array([[int(x) for x in row] for row in golden("window_sink_visibility_s6_w3_k1.txt")])
    vis = (oracle.window_mask(np.arange(6), 6, 3, 1) == 0).astype(int)
    assert np.array_equal(vis, table)


def test_window_of_one_returns_own_value():
    """W = 1 without sinks: every query sees only its own key, so the output row is v_p exactly."""
    rng = np.random.default_rng(31)
    B, T, Nh, Nkv, D = 1, 12, 2, 1, 8
    q, k, v = _rand(rng, B, T, Nh, D), _rand(rng, B, T, Nkv, D), _rand(rng, B, T, Nkv, D)
    got = oracle.prefill_chunk(q, k, v, [0], window=1)
    for h in range(Nh):
        np.testing.assert_array_equal(got[0, :, h], v[0, :, 0])


@pytest.mark.parametrize("window,sinks", [(40, 0), (12, 40), (5, 12)])
def test_wide_window_or_all_sinks_is_causal(window, sinks):
    """A window covering the whole prefix, or sinks covering it, leaves the causal mask; a narrow
    window differs from it (the mask is not a no-op)."""
    rng = np.random.default_rng(32)
    B, T, Nh, Nkv, D = 2, 12, 2, 2, 8
    q, k, v = _rand(rng, B, T, Nh, D), _rand(rng, B, T, Nkv, D), _rand(rng, B, T, Nkv, D)
    full = oracle.prefill(q, k, v)
    got = oracle.prefill_chunk(q, k, v, [0, 0], window=window, sinks=sinks)
    np.testing.assert_allclose(got, full, rtol=1e-12, atol=1e-13)
    narrow = oracle.prefill_chunk(q, k, v, [0, 0], window=3, sinks=1)
    assert np.abs(narrow - full).max() > 1e-3


# ------------------------------------------------------------- partial and decoupled RoPE --
def test_partial_rotary_rotates_only_its_span():
    """rot_dims = D_r: the span is rotated exactly as a D_r-dim head (frequencies base^(-2i/D_r)),
    the rest passes through; the full span is the default rotation."""
    rng = np.random.default_rng(41)
    x = _rand(rng, 2, 9, 3, 16)
    pos = np.arange(9) * 7
    np.testing.assert_array_equal(oracle.rope_rotate(x, pos, 1e4, rot_dims=16), oracle.rope_rotate(x, pos, 1e4))
    for inter in (False, True):
        got = oracle.rope_rotate(x, pos, 1e4, interleaved=inter, rot_dims=8)
        np.testing.assert_allclose(got[..., :8], oracle.rope_rotate(x[..., :8], pos, 1e4, interleaved=inter),
                                   rtol=0, atol=1e-14)
        np.testing.assert_array_equal(got[..., 8:], x[..., 8:])
        got = oracle.rope_rotate(x, pos, 1e4, interleaved=inter, rot_dims=4, rot_offset=12)
        np.testing.assert_allclose(got[..., 12:], oracle.rope_rotate(x[..., 12:], pos, 1e4, interleaved=inter),
                                   rtol=0, atol=1e-14)
        np.testing.assert_array_equal(got[..., :12], x[..., :12])


def test_mla_decoupled_rope_absorbed_equals_per_head():
    """[P4] slide 06: RoPE acts only on the 64-dim q^R / k^R block, so it cannot be absorbed; the
    absorbed decode with q^R rotated at ctx-1 (cache rows holding rotated k^R) equals per-head
    attention with q^R and k^R rotated at their positions."""
    rng = np.random.default_rng(42)
    H, T, dc, dr, dh, theta = 4, 21, 32, 8, 16, 1e4
    c = _rand(rng, T, dc) * 0.2
    kr = _rand(rng, T, dr)
    qc, qr = _rand(rng, H, dh) * 0.3, _rand(rng, H, dr)
    w_uk, w_uv = _rand(rng, H, dh, dc) * 0.2, _rand(rng, H, dh, dc) * 0.2
    scale = 1.0 / math.sqrt(dh + dr)
    kr_rot = oracle.rope_rotate(kr[None, :, None, :], np.arange(T), theta)[0, :, 0]
    qr_rot = oracle.rope_rotate(qr[None, None], [T - 1], theta)[0, 0]
    ref = np.stack([
        oracle.head_attention(np.concatenate([qc[h], qr_rot[h]])[None],
                              np.concatenate([c @ w_uk[h].T, kr_rot], axis=1), c @ w_uv[h].T, scale)[0]
        for h in range(H)])
    q_abs = np.concatenate([np.einsum("hd,hdc->hc", qc, w_uk), qr], axis=1)[None]
    row = np.concatenate([c, kr_rot], axis=1)[None, :, None, :]
    lat = oracle.decode(q_abs, row, row[..., :dc], np.array([T]), scale=scale, rope_theta=theta)[0]
    np.testing.assert_allclose(np.einsum("hdc,hc->hd", w_uv, lat), ref, rtol=1e-10, atol=1e-12)


def test_mla_non_absorbed_prefill_equals_absorbed_decode():
    """[P4] slide 06: prefill keeps W_UK / W_UV un-absorbed, per head q = [q^C ; q^R] and
    k = [k^C ; k^R] (k^R shared by the heads) with v = c W_UV; RoPE only on the
    decoupled block. Row t of that causal prefill equals the absorbed decode of query t over the
    first t + 1 cache rows [c ; rotated k^R], mapped back through W_UV."""
    rng = np.random.default_rng(43)
    H, T, dc, dr, dh, theta = 3, 11, 24, 8, 16, 1e4
    c = _rand(rng, T, dc) * 0.2
    kr = _rand(rng, T, dr)
    qc, qr = _rand(rng, T, H, dh) * 0.3, _rand(rng, T, H, dr)
    w_uk, w_uv = _rand(rng, H, dh, dc) * 0.2, _rand(rng, H, dh, dc) * 0.2
    scale = 1.0 / math.sqrt(dh + dr)
    q = np.concatenate([qc, qr], axis=2)[None]  # [1, T, H, dh + dr]
    k = np.concatenate([np.einsum("tc,hdc->thd", c, w_uk), np.repeat(kr[:, None], H, axis=1)], axis=2)[None]
    v = np.einsum("tc,hdc->thd", c, w_uv)[None]  # [1, T, H, dh]
    got = oracle.prefill(q, k, v, scale=scale, rope_theta=theta)[0]  # [T, H, dh]
    kr_rot = oracle.rope_rotate(kr[None, :, None, :], np.arange(T), theta)[0, :, 0]
    row = np.concatenate([c, kr_rot], axis=1)[None, :, None, :]
    for t in range(T):
        q_abs = np.concatenate([np.einsum("hd,hdc->hc", qc[t], w_uk), qr[t]], axis=1)[None]
        lat = oracle.decode(q_abs, row, row[..., :dc], np.array([t + 1]), scale=scale, rope_theta=theta)[0]
        np.testing.assert_allclose(got[t], np.einsum("hdc,hc->hd", w_uv, lat), rtol=1e-10, atol=1e-12)
    # the rotation reaches only the decoupled block: without RoPE on it the result differs
    plain = oracle.prefill(q, k, v, scale=scale)[0]
    assert np.abs(plain - got).max() > 1e-3
    np.testing.assert_array_equal(plain[0], v[0, 0])  # position 0: the only key, no rotation
