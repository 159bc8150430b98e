"""fp64 CPU oracle for the causal-attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the CPU-baseline leg
of bench.py, never by the product library. See oracle/attention.py for the definitions and
their citations.
"""
from .attention import (  # noqa: F401
    attention_weights,
    causal_mask,
    decode,
    head_attention,
    kv_head_of,
    prefill,
    prefill_chunk,
    prefill_rows,
    rope_angles,
    rope_inv_freq,
    rope_rotate,
    softmax_rows,
    window_mask,
)
