"""fp64 CPU oracle: plain, slow, materialising definition of causal scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do. It shares no code with
the HIP library and receives its inputs from the seeded generators in ``synth.py``.

Every step follows the plain definition written on the pages; none of the tiling, online
softmax or split-KV machinery of the GPU path appears here (exact attention has one result:
"Transformer 架构完全深度解析" §十三 states the tiled method is mathematically identical).

Sources (cited by page title and section):
  [P1] "2.7 Transformer Decoder Block完整解析" (ningzhengsheng.cn)
  [P2] "Transformer 架构快速入门" (liumengxuan04.github.io)
  [P3] "Transformer 架构完全深度解析" (tufusi.com)
  [P4] "Transformer 与 LLM：结构、实现与算量" (arganzheng.life slides)

Where the pages are silent or disagree, the reading taken is stated next to the step it affects.

Parity pins: every function here is pinned by tests/test_oracle.py against printed values,
closed forms or invariants; no function is "parity unpinned". The page's own d=4, T=3 inputs
are not in the text, so that example is pinned through a constructed case whose closed form
rounds to the printed weights.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# RoPE  ([P1] §4 precompute/apply; [P2] §8.2 frequencies, §8.3 rotation; [P3] §七)
# ---------------------------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Pair frequencies theta_i = base^(-2i/D) for i = 0 .. D/2-1 ([P1] §4, [P2] §8.2).

    The index is 0-based (theta_0 = 1), as in [P1]'s table code; [P4] slide 07's count of 14
    unfinished low-frequency pairs at 8K (D=128, base 1e4) fixes this choice.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * i / head_dim)


def rope_angles(positions, head_dim: int, theta: float) -> np.ndarray:
    """Angle m * theta_i for every position m and pair i ([P2] §8.2): shape positions.shape + (D/2,)."""
    return _f64(positions)[..., None] * rope_inv_freq(head_dim, theta)


def rope_rotate(x, positions, theta: float, interleaved: bool = False, rot_dims: int | None = None,
                rot_offset: int = 0) -> np.ndarray:
    """Rotate every head vector of x [B, S, N, D] by its position's angles, in fp64.

    positions: [S] (shared by the batch) or [B, S].
    Half-split pairing (default) rotates (x_i, x_{i+D/2}) as in [P1] §4's apply_rope:
        (x_i cos a - x_{i+D/2} sin a,  x_i sin a + x_{i+D/2} cos a).
    interleaved=True rotates adjacent pairs (x_{2i}, x_{2i+1}) with the same 2x2 rotation
    ([P2] §8.3, [P3] §七). [P2] §8.1 notes that either pairing works when used consistently.
    rot_dims = D_r < D rotates only the D_r dims starting at rot_offset, with frequencies
    base^(-2i/D_r) ([P2] §8.2: D_r is the rotary dimension, possibly a part of the head); the other
    dims pass unchanged. Reading: the rotary span is the leading D_r dims (rot_offset = 0), or the
    decoupled k^R / q^R block of MLA ([P4] slide 06), which sits after the 512 latent dims.
    """
    x = _f64(x)
    B, S, N, D = x.shape
    Dr = D if rot_dims is None else int(rot_dims)
    pos = np.broadcast_to(_f64(positions), (B, S))
    ang = rope_angles(pos, Dr, theta)[:, :, None, :]  # [B, S, 1, D_r/2]
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    xr = x[..., rot_offset:rot_offset + Dr]
    rr = out[..., rot_offset:rot_offset + Dr]
    if interleaved:
        a, b = xr[..., 0::2], xr[..., 1::2]
        rr[..., 0::2] = a * c - b * s
        rr[..., 1::2] = a * s + b * c
    else:
        h = Dr // 2
        a, b = xr[..., :h], xr[..., h:]
        rr[..., :h] = a * c - b * s
        rr[..., h:] = a * s + b * c
    return out


# ---------------------------------------------------------------------------------------------
# Mask, softmax, one head  ([P1] §3, §4; [P2] §4.2-4.5; [P3] §五)
# ---------------------------------------------------------------------------------------------
def causal_mask(q_positions, n_keys: int) -> np.ndarray:
    """Additive causal mask M[r, j] = -inf where key j lies after the query's position, else 0.

    For q_positions = 0..S-1 this is the S x S matrix printed in [P1] §3.2 / §3.3.
    """
    j = np.arange(n_keys)
    return np.where(j[None, :] > np.asarray(q_positions)[:, None], -np.inf, 0.0)


def window_mask(q_positions, n_keys: int, window: int, sinks: int = 0) -> np.ndarray:
    """Causal sliding-window mask with attention sinks ([P4] slide 07: a window of W keys, plus the
    first few tokens kept). Reading: the query at position p sees keys p-W+1 .. p (its own key
    included, W keys at most) and the sink keys 0 .. sinks-1; every other key is masked with -inf.
    """
    j = np.arange(n_keys)[None, :]
    p = np.asarray(q_positions)[:, None]
    hidden = (j > p) | ((j < p - window + 1) & (j >= sinks))
    return np.where(hidden, -np.inf, 0.0)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax over the key axis ([P2] §4.4, [P3] §五 step 4): exp(s - max) / sum."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_weights(q, k, scale: float, mask=None) -> np.ndarray:
    """A = softmax(scale * q k^T + M) for one head: q [R, D], k [T, D] -> [R, T] ([P2] §4.2-4.4)."""
    s = np.float64(scale) * (_f64(q) @ _f64(k).T)
    if mask is not None:
        s = s + mask
    return softmax_rows(s)


def head_attention(q, k, v, scale: float, mask=None) -> np.ndarray:
    """O = A v for one head ([P2] §4.5: o_m = sum_n A_mn v_n): returns [R, Dv]."""
    return attention_weights(q, k, scale, mask) @ _f64(v)


# ---------------------------------------------------------------------------------------------
# Prefill: all positions of a sequence at once, GQA head sharing ([P2] §6.3)
# ---------------------------------------------------------------------------------------------
def kv_head_of(h: int, n_heads: int, n_kv_heads: int) -> int:
    """Query head h reads KV head h // G with G = N_h / N_kv consecutive query heads per group
    ([P2] §6.3: heads 1-4 -> KV 1, ..., 29-32 -> KV 8, written here 0-based)."""
    return h // (n_heads // n_kv_heads)


def prefill_rows(q, k, v, b: int, h: int, rows, *, causal: bool = True, scale: float | None = None,
                 rope_theta: float = 0.0) -> np.ndarray:
    """Output rows out[b, rows, h, :] of causal self-attention over one sequence, in fp64.

    q [B, S, Nh, D], k/v [B, S, Nkv, D] (any float dtype; values are taken exactly).
    Query and key positions are 0..S-1 ([P1] §4 uses arange(seq_len)). RoPE, when
    rope_theta > 0, rotates q and k (not v: [P1] §2, [P2] §8.5) before the scores.
    The full score row over all S keys is materialised and masked with -inf ([P1] §3.3).
    MLA's non-absorbed prefill ([P4] slide 06) has v narrower than q/k: q = [q^C ; q^R],
    k = [k^C ; k^R] with v of the width of q^C. There RoPE touches only the decoupled block,
    the last D - Dv dims (half-split pairs, frequencies base^(-2i/(D - Dv))), as in decode.
    """
    B, S, Nh, D = q.shape
    Nkv = k.shape[2]
    Dv = v.shape[3]
    g = kv_head_of(h, Nh, Nkv)
    rows = np.asarray(rows, dtype=np.int64)
    if scale is None:
        scale = 1.0 / np.sqrt(D)  # [P2] §4.3: divide by the per-head dimension
    qh = _f64(q[b:b + 1, rows, h:h + 1, :])  # [1, R, 1, D]
    kh = _f64(k[b:b + 1, :, g:g + 1, :])  # [1, S, 1, D]
    if rope_theta > 0:
        span = {} if Dv == D else {"rot_dims": D - Dv, "rot_offset": Dv}
        qh = rope_rotate(qh, rows, rope_theta, **span)
        kh = rope_rotate(kh, np.arange(S), rope_theta, **span)
    mask = causal_mask(rows, S) if causal else None
    return head_attention(qh[0, :, 0, :], kh[0, :, 0, :], v[b, :, g, :], scale, mask)


def prefill(q, k, v, *, causal: bool = True, scale: float | None = None, rope_theta: float = 0.0) -> np.ndarray:
    """Full prefill output [B, S, Nh, Dv] in fp64 (every (b, h) independently)."""
    B, S, Nh, _ = q.shape
    out = np.empty((B, S, Nh, v.shape[3]), dtype=np.float64)
    rows = np.arange(S)
    for b in range(B):
        for h in range(Nh):
            out[b, :, h, :] = prefill_rows(q, k, v, b, h, rows, causal=causal, scale=scale, rope_theta=rope_theta)
    return out


# ---------------------------------------------------------------------------------------------
# Prefill against a KV cache: a chunk of new tokens after a cached prefix ([P3] §九, [P4] slide 07)
# ---------------------------------------------------------------------------------------------
def prefill_chunk(q, k, v, q_start, *, causal: bool = True, scale: float | None = None,
                  rope_theta: float = 0.0, window: int = 0, sinks: int = 0, rope_interleaved: bool = False,
                  rope_dims: int | None = None) -> np.ndarray:
    """Output [B, S, Nh, Dv] of S new queries per sequence that follow q_start[b] cached tokens.

    q [B, S, Nh, D]: query s of sequence b has absolute position q_start[b] + s.
    k, v [B, T, Nkv, D]: the sequence's keys/values at positions 0 .. T-1 (un-rotated);
    positions 0 .. q_start[b]+S-1 are used, i.e. the chunk's own K/V are appended before the
    queries attend ([P3] §九: concat to the cache, then attend).
    Reading (the pages only draw square masks, [P1] §3.1): the causal rule "no key after the
    query" is applied in absolute positions, so the query at position p sees keys 0 .. p; the
    chunk's last query sees every key (the mask is the square one's bottom-right block).
    RoPE, when rope_theta > 0, rotates q and k at their absolute positions ([P1] §4).
    window > 0 (with causal) replaces the causal mask by window_mask(..., window, sinks).
    rope_interleaved / rope_dims select the pairing and the rotary dimension (see rope_rotate).
    """
    B, S, Nh, D = q.shape
    Nkv = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.empty((B, S, Nh, v.shape[3]), dtype=np.float64)
    for b in range(B):
        n = int(q_start[b]) + S
        pos = int(q_start[b]) + np.arange(S)
        for h in range(Nh):
            g = kv_head_of(h, Nh, Nkv)
            qh = _f64(q[b:b + 1, :, h:h + 1, :])
            kh = _f64(k[b:b + 1, :n, g:g + 1, :])
            if rope_theta > 0:
                qh = rope_rotate(qh, pos, rope_theta, rope_interleaved, rope_dims)
                kh = rope_rotate(kh, np.arange(n), rope_theta, rope_interleaved, rope_dims)
            if window > 0:
                mask = window_mask(pos, n, window, sinks)
            else:
                mask = causal_mask(pos, n) if causal else None
            out[b, :, h, :] = head_attention(qh[0, :, 0, :], kh[0, :, 0, :], v[b, :n, g, :], scale, mask)
    return out


# ---------------------------------------------------------------------------------------------
# KV-cache decode ([P2] §13.2, [P3] §九) and the MLA-absorbed form ([P4] slide 06)
# ---------------------------------------------------------------------------------------------
def decode(q, kcache, vcache, ctx_lens, *, scale: float | None = None, rope_theta: float = 0.0) -> np.ndarray:
    """One new query token per sequence attends to every cached key of its KV head.

    q [B, Nh, Dqk]; kcache [B, T, Nkv, Dqk]; vcache [B, T, Nkv, Dv]; ctx_lens [B].
    ctx_lens[b] counts the keys 0..ctx_b-1, the new token included: [P3] §九 appends the new
    K/V before attending, so no mask is applied. The cache holds already-rotated keys ([P3] §七:
    cached keys carry their position); with rope_theta > 0 the query is rotated at position
    ctx_b - 1. For the MLA-absorbed form pass vcache = kcache[..., :Dv], i.e. V is the latent
    part c^KV of the same cached row ([P4] slide 06); there RoPE touches only the decoupled q^R
    block (the last Dqk - Dv dims, half-split pairs, frequencies base^(-2i/(Dqk - Dv))).
    Returns [B, Nh, Dv] in fp64.
    """
    B, Nh, Dqk = q.shape
    Nkv = kcache.shape[2]
    Dv = vcache.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(Dqk)
    out = np.empty((B, Nh, Dv), dtype=np.float64)
    for b in range(B):
        c = int(ctx_lens[b])
        for h in range(Nh):
            g = kv_head_of(h, Nh, Nkv)
            qh = _f64(q[b, h, :])[None, None, None, :]
            if rope_theta > 0:
                if Dqk != Dv:  # MLA: decoupled RoPE block after the latent dims
                    qh = rope_rotate(qh, [c - 1], rope_theta, rot_dims=Dqk - Dv, rot_offset=Dv)
                else:
                    qh = rope_rotate(qh, [c - 1], rope_theta)
            out[b, h, :] = head_attention(qh[0, 0], kcache[b, :c, g, :], vcache[b, :c, g, :], scale)[0]
    return out
