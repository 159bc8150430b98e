"""Algorithmic FLOP and byte counts used to place measured times on the MI355X roofline.

Pure arithmetic on sizes; no attention math. Conventions:
- A score pair (query i, key j) costs 2*Dqk FLOPs for q.k and 2*Dv FLOPs for the P.V update
  (2 FLOPs per multiply-add). Causal prefill counts only the S(S+1)/2 unmasked pairs, since
  the method skips the masked ones ("2.7 Transformer Decoder Block完整解析" §3.3).
- Decode bytes are the compulsory ones: the cached K/V rows each query actually needs, plus q
  and out. A cached row that serves as both K and V (the MLA latent row) is counted once.
  Split-KV partial results are workspace traffic and are not algorithmic bytes.
"""
from __future__ import annotations

import numpy as np

# MI355X published peaks (dense).
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP32_VECTOR_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: int) -> int:
    """K and V rows of every layer: 2 * L * n_kv * d_head * bytes
    ("Transformer 与 LLM：结构、实现与算量" slide 02 and slide 06)."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def mla_bytes_per_token(layers: int, row_elems: int, bytes_per_elem: int) -> int:
    """MLA caches one shared row [c^KV ; k^R] per token and layer, no factor 2 (slide 06)."""
    return layers * row_elems * bytes_per_elem


def logits_bytes(seq: int, heads: int, bytes_per_elem: int) -> int:
    """Size of a materialised S = Q K^T for one layer (slide 06: 8K context, 32 heads, BF16)."""
    return seq * seq * heads * bytes_per_elem


def mla_absorbed_intensity(heads: int = 128, d_qk: int = 576, d_v: int = 512, bytes_per_elem: int = 2) -> float:
    """FLOPs per cache byte of absorbed MLA decode: every cached row feeds all heads' q.k and P.V."""
    return 2.0 * heads * (d_qk + d_v) / (d_qk * bytes_per_elem)


def mla_absorbed_flop_ratio(d_qk_abs: int = 576, d_v_abs: int = 512, d_qk: int = 192, d_v: int = 128) -> float:
    """Attention FLOPs per (head, key) of the absorbed form over the non-absorbed one."""
    return (d_qk_abs + d_v_abs) / (d_qk + d_v)


def prefill_pairs(S: int, causal: bool) -> int:
    return S * (S + 1) // 2 if causal else S * S


def prefill_flops(B: int, S: int, Nh: int, Dh: int, causal: bool = True, Dv: int | None = None) -> int:
    """2 FLOP per multiply-add of Q K^T (Dh per pair) and of P V (Dv per pair, Dv = Dh unless given:
    MLA's non-absorbed prefill has Dh = 192, Dv = 128) over the unmasked (query, key) pairs."""
    dv = Dh if Dv is None else Dv
    return 2 * (Dh + dv) * B * Nh * prefill_pairs(S, causal)


def prefill_bytes(B: int, S: int, Nh: int, Nkv: int, Dh: int, bytes_per_elem: int) -> int:
    """q, k, v read once and out written once."""
    return (2 * B * S * Nh * Dh + 2 * B * S * Nkv * Dh) * bytes_per_elem


def decode_flops(ctx_lens, Nh: int, Dqk: int, Dv: int) -> int:
    return int(np.sum(np.asarray(ctx_lens, dtype=np.int64))) * Nh * 2 * (Dqk + Dv)


def decode_bytes(ctx_lens, B: int, Nh: int, Nkv: int, Dqk: int, Dv: int, bytes_per_elem: int,
                 shared_row: bool = False) -> int:
    tokens = int(np.sum(np.asarray(ctx_lens, dtype=np.int64)))
    row = Dqk if shared_row else Dqk + Dv
    return (tokens * Nkv * row + B * Nh * (Dqk + Dv)) * bytes_per_elem
