"""Seeded synthetic inputs for the causal-attention workloads.

This module only draws numbers and rounds them to the storage type; it holds none of the
attention arithmetic. Both the fp64 CPU oracle (``oracle/``) and the HIP path receive the very
same arrays from here, so neither side ever produces the other's inputs.

Generator: ``numpy.random.default_rng(SeedSequence([workload_id, tensor_id]))`` (PCG64),
``standard_normal`` in fp32, then round-to-nearest-even to bf16 where the workload is bf16.
Tensor ids: q=0, k=1, v=2, ctx_lens=3 (for the MLA cache the single latent cache is id 1).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_CTX = 0, 1, 2, 3


# --------------------------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only; bf16 -> fp32 is exact)
# --------------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 with round-to-nearest-even; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), rounded).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(workload_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(workload_id), int(tensor_id)]))


def normal(workload_id: int, tensor_id: int, shape, dtype: str) -> np.ndarray:
    """N(0,1) tensor. dtype 'f32' returns float32; 'bf16' returns uint16 bf16 bit patterns."""
    x = _rng(workload_id, tensor_id).standard_normal(size=tuple(shape), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def uniform_ctx_lens(workload_id: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn uniformly from the closed range [lo, hi] (int32)."""
    return _rng(workload_id, TENSOR_CTX).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of a stored tensor as fp32 (exact for both storage types)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


# --------------------------------------------------------------------------------------------
# Workloads: shapes of the models the pages discuss (GPT-2-small, Llama-3-8B, DeepSeek-V3 MLA)
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Prefill:
    wid: int
    name: str
    B: int
    S: int
    Nh: int
    Nkv: int
    Dh: int
    dtype: str
    rope_theta: float
    causal: bool = True
    Dv: int = 0  # head dim of v / out when it differs from the q/k head dim Dh (MLA prefill)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dh)

    @property
    def dv(self) -> int:
        return self.Dv or self.Dh

    def inputs(self):
        q = normal(self.wid, TENSOR_Q, (self.B, self.S, self.Nh, self.Dh), self.dtype)
        k = normal(self.wid, TENSOR_K, (self.B, self.S, self.Nkv, self.Dh), self.dtype)
        v = normal(self.wid, TENSOR_V, (self.B, self.S, self.Nkv, self.dv), self.dtype)
        return q, k, v


@dataclasses.dataclass(frozen=True)
class Decode:
    wid: int
    name: str
    B: int
    Nh: int
    Nkv: int
    Dqk: int
    Dv: int
    max_ctx: int
    ctx_lo: int
    ctx_hi: int
    dtype: str
    scale: float
    mla: bool = False  # V aliases the first Dv dims of the single cached K row

    def ctx_lens(self) -> np.ndarray:
        if self.ctx_lo == self.ctx_hi:
            return np.full(self.B, self.ctx_lo, dtype=np.int32)
        return uniform_ctx_lens(self.wid, self.B, self.ctx_lo, self.ctx_hi)

    def inputs(self):
        """q [B,Nh,Dqk]; kcache [B,max_ctx,Nkv,Dqk]; vcache [B,max_ctx,Nkv,Dv] (None for MLA)."""
        q = normal(self.wid, TENSOR_Q, (self.B, self.Nh, self.Dqk), self.dtype)
        k = normal(self.wid, TENSOR_K, (self.B, self.max_ctx, self.Nkv, self.Dqk), self.dtype)
        v = None if self.mla else normal(self.wid, TENSOR_V, (self.B, self.max_ctx, self.Nkv, self.Dv), self.dtype)
        return q, k, v, self.ctx_lens()


TINY_F32 = Prefill(1, "tiny causal MHA fp32", B=1, S=128, Nh=4, Nkv=4, Dh=16, dtype="f32", rope_theta=10000.0)
GPT2_PREFILL = Prefill(2, "GPT-2-small causal MHA prefill", B=8, S=1024, Nh=12, Nkv=12, Dh=64, dtype="bf16",
                       rope_theta=0.0)
LLAMA3_PREFILL = Prefill(3, "Llama-3-8B GQA causal prefill", B=4, S=8192, Nh=32, Nkv=8, Dh=128, dtype="bf16",
                         rope_theta=500000.0)
LLAMA3_DECODE = Decode(4, "Llama-3-8B GQA KV-cache decode", B=64, Nh=32, Nkv=8, Dqk=128, Dv=128, max_ctx=8192,
                       ctx_lo=1024, ctx_hi=8192, dtype="bf16", scale=1.0 / math.sqrt(128))
MLA_DECODE = Decode(5, "MLA-absorbed decode (MQA form)", B=32, Nh=128, Nkv=1, Dqk=576, Dv=512, max_ctx=4096,
                    ctx_lo=4096, ctx_hi=4096, dtype="bf16", scale=1.0 / math.sqrt(192), mla=True)
# DeepSeek-V3-shaped non-absorbed MLA prefill: per head q/k = [128 ; 64 decoupled RoPE] dims, v 128
MLA_PREFILL = Prefill(6, "MLA non-absorbed causal prefill", B=1, S=4096, Nh=128, Nkv=128, Dh=192, Dv=128,
                      dtype="bf16", rope_theta=10000.0)

WORKLOADS = {w.wid: w for w in (TINY_F32, GPT2_PREFILL, LLAMA3_PREFILL, LLAMA3_DECODE, MLA_DECODE, MLA_PREFILL)}
