"""ctypes binding of libattn_gfx950.so: argument marshalling only.

Every step of the computation runs in the HIP library; this module turns torch tensors into
device pointers, sizes the outputs and workspaces (torch allocates them), and passes torch's
current HIP stream. There is no fallback: if the shared library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_gfx950.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTS = (
    "attn_status_str",
    "attn_prefill_workspace_bytes",
    "attn_prefill",
    "attn_decode_workspace_bytes",
    "attn_decode",
    "rope_apply",
    "attn_prefill_cached_workspace_bytes",
    "attn_prefill_cached",
    "attn_kv_append",
    "attn_prefill_mla_workspace_bytes",
    "attn_prefill_mla",
    "attn_decode_noalloc_max_bytes",
    "attn_decode_noalloc",
    "attn_set_kernel_events",
)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed: {status_str(status)}")


def load() -> ctypes.CDLL:
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m causal_head_attention_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_float, c_size, c_vp, c_ll = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_longlong
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [c_int]
    lib.attn_prefill_workspace_bytes.restype = c_size
    lib.attn_prefill_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_float, c_int]
    lib.attn_prefill.restype = c_int
    lib.attn_prefill.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_float,
                                 c_int, c_vp, c_size, c_vp]
    lib.attn_decode_workspace_bytes.restype = c_size
    lib.attn_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int]
    lib.attn_decode.restype = c_int
    lib.attn_decode.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_ll, c_ll,
                                c_float, c_float, c_int, c_vp, c_size, c_vp]
    lib.rope_apply.restype = c_int
    lib.rope_apply.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_int, c_float, c_int, c_int, c_vp]
    lib.attn_prefill_cached_workspace_bytes.restype = c_size
    lib.attn_prefill_cached_workspace_bytes.argtypes = [c_int, c_int, c_float]
    lib.attn_prefill_cached.restype = c_int
    lib.attn_prefill_cached.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_ll,
                                        c_float, c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_vp, c_size,
                                        c_vp]
    lib.attn_kv_append.restype = c_int
    lib.attn_kv_append.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_ll, c_ll,
                                   c_float, c_int, c_int, c_int, c_vp]
    lib.attn_prefill_mla_workspace_bytes.restype = c_size
    lib.attn_prefill_mla_workspace_bytes.argtypes = [c_int, c_int, c_int, c_float]
    lib.attn_prefill_mla.restype = c_int
    lib.attn_prefill_mla.argtypes = [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_float, c_int, c_float,
                                     c_vp, c_size, c_vp]
    lib.attn_decode_noalloc_max_bytes.restype = c_size
    lib.attn_decode_noalloc_max_bytes.argtypes = []
    lib.attn_decode_noalloc.restype = c_int
    lib.attn_decode_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_ll,
                                        c_ll, c_float, c_float, c_int, c_vp]
    lib.attn_set_kernel_events.restype = c_int
    lib.attn_set_kernel_events.argtypes = [c_vp, c_vp]
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().attn_status_str(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != ATTN_OK:
        raise AttnError(status, what)


# ------------------------------------------------------------------------------ torch side ----
def _torch():
    import torch  # noqa: WPS433 (torch is plumbing: device memory and streams)
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_ptr(dev) -> int:
    return _torch().cuda.current_stream(dev).cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_out(out, shape, dtype, device):
    """A caller-supplied output must be exactly what the kernel writes: shape, dtype, device, dense."""
    if not out.is_cuda or out.device != device:
        raise ValueError(f"out must live on {device}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.dtype != dtype:
        raise TypeError(f"out must be {dtype}, got {out.dtype}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    return out


def _workspace(ws, need: int, device):
    """(pointer, bytes) of a workspace: torch allocates it when the caller gives none; a given one
    must be a dense buffer on the same device (its size is checked by the library)."""
    torch = _torch()
    if ws is None:
        if need <= 0:
            return None, 0
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    if not ws.is_cuda or ws.device != device:
        raise ValueError(f"workspace must live on {device}")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def prefill_workspace_bytes(B: int, S: int, Nkv: int, Dh: int, rope_theta: float, dtype: int) -> int:
    return int(load().attn_prefill_workspace_bytes(B, S, Nkv, Dh, float(rope_theta), dtype))


def decode_workspace_bytes(B: int, Nh: int, Nkv: int, Dqk: int, Dv: int, max_ctx: int, dtype: int) -> int:
    return int(load().attn_decode_workspace_bytes(B, Nh, Nkv, Dqk, Dv, max_ctx, dtype))


def prefill(q, k, v, *, rope_theta: float = 0.0, causal: bool = True, scale: float | None = None, out=None,
            workspace=None):
    """Causal (or full) attention over [B, S, N, Dh] BSHD tensors; returns out [B, S, Nh, Dh]."""
    torch = _torch()
    _need_cuda(q, k, v)
    B, S, Nh, Dh = q.shape
    Nkv = k.shape[2]
    if k.shape != (B, S, Nkv, Dh) or v.shape != (B, S, Nkv, Dh):
        raise ValueError("q/k/v shapes disagree")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    out = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    ws_ptr, ws_len = _workspace(workspace, prefill_workspace_bytes(B, S, Nkv, Dh, rope_theta, dt), q.device)
    st = load().attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, Nh, Nkv, Dh,
                             float(rope_theta), 1 if causal else 0, float(scale or 0.0), dt, ws_ptr, ws_len,
                             _stream_ptr(q.device))
    _check(st, "attn_prefill")
    return out


def prefill_mla_workspace_bytes(B: int, S: int, Nkv: int, rope_theta: float) -> int:
    return int(load().attn_prefill_mla_workspace_bytes(B, S, Nkv, float(rope_theta)))


def prefill_mla(q, k, v, *, rope_theta: float = 0.0, causal: bool = True, scale: float | None = None, out=None,
                workspace=None):
    """MLA's non-absorbed prefill: q [B, S, Nh, 192], k [B, S, Nkv, 192], v [B, S, Nkv, 128]
    (bf16); RoPE on dims 128..191 only. Returns out [B, S, Nh, 128]."""
    torch = _torch()
    _need_cuda(q, k, v)
    B, S, Nh, Dqk = q.shape
    Nkv = k.shape[2]
    if Dqk != 192 or k.shape != (B, S, Nkv, 192) or v.shape != (B, S, Nkv, 128):
        raise ValueError("MLA prefill expects q/k [..., 192] and v [..., 128] over the same B, S")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("MLA prefill takes bf16 q, k, v")
    if out is None:
        out = torch.empty((B, S, Nh, 128), dtype=q.dtype, device=q.device)
    _check_out(out, (B, S, Nh, 128), q.dtype, q.device)
    ws_ptr, ws_len = _workspace(workspace, prefill_mla_workspace_bytes(B, S, Nkv, rope_theta), q.device)
    st = load().attn_prefill_mla(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, S, Nh, Nkv,
                                 float(rope_theta), 1 if causal else 0, float(scale or 0.0), ws_ptr, ws_len,
                                 _stream_ptr(q.device))
    _check(st, "attn_prefill_mla")
    return out


def decode(q, kcache, vcache, ctx_lens, *, scale: float | None = None, rope_theta: float = 0.0, out=None,
           workspace=None):
    """One query token per sequence against a KV cache.

    q [B, Nh, Dqk]; kcache [B, max_ctx, Nkv, Dqk]-shaped (last dim may be a view of a wider row:
    its row pitch is taken from the stride); vcache [B, max_ctx, Nkv, Dv] likewise, possibly a
    view into kcache's rows (MLA: vcache = kcache[..., :512]); ctx_lens int32 [B] on the GPU.
    Returns out [B, Nh, Dv] (bf16).
    """
    torch = _torch()
    _need_cuda(q, ctx_lens)
    for t in (kcache, vcache):
        if not t.is_cuda:
            raise ValueError("caches must live on the GPU")
        B_, T_, N_, D_ = t.shape
        if t.stride(3) != 1 or t.stride(1) != N_ * t.stride(2) or t.stride(0) != T_ * t.stride(1):
            raise ValueError("cache must be [B, max_ctx, Nkv, row] with a dense row pitch")
    B, Nh, Dqk = q.shape
    _, max_ctx, Nkv, Dk = kcache.shape
    Dv = vcache.shape[3]
    if Dk != Dqk or vcache.shape[:3] != kcache.shape[:3]:
        raise ValueError("cache shapes disagree with q")
    if ctx_lens.dtype != torch.int32 or ctx_lens.shape != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    dt = _dtype_code(q)
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    if out is None:
        out = torch.empty((B, Nh, Dv), dtype=q.dtype, device=q.device)
    _check_out(out, (B, Nh, Dv), q.dtype, q.device)
    ws_ptr, ws_len = _workspace(workspace, decode_workspace_bytes(B, Nh, Nkv, Dqk, Dv, max_ctx, dt),
                                q.device)
    st = load().attn_decode(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), ctx_lens.data_ptr(), out.data_ptr(),
                            B, Nh, Nkv, Dqk, Dv, max_ctx, kcache.stride(2), vcache.stride(2), float(rope_theta),
                            float(scale or 0.0), dt, ws_ptr, ws_len, _stream_ptr(q.device))
    _check(st, "attn_decode")
    return out


def decode_noalloc(q, kcache, vcache, ctx_lens, *, scale: float | None = None, rope_theta: float = 0.0, out):
    """attn_decode without a workspace (the library's static per-GPU scratch holds the split
    partials): for callers that cannot allocate, such as code under graph capture. `out` must be
    given ([B, Nh, Dv], the dtype of q); arguments are those of decode(). Calls that overlap in
    time on one GPU race on the scratch."""
    _need_cuda(q, ctx_lens)
    for t in (kcache, vcache):
        if not t.is_cuda:
            raise ValueError("caches must live on the GPU")
        B_, T_, N_, D_ = t.shape
        if t.stride(3) != 1 or t.stride(1) != N_ * t.stride(2) or t.stride(0) != T_ * t.stride(1):
            raise ValueError("cache must be [B, max_ctx, Nkv, row] with a dense row pitch")
    B, Nh, Dqk = q.shape
    _, max_ctx, Nkv, Dk = kcache.shape
    Dv = vcache.shape[3]
    if Dk != Dqk or vcache.shape[:3] != kcache.shape[:3]:
        raise ValueError("cache shapes disagree with q")
    if ctx_lens.dtype != _torch().int32 or ctx_lens.shape != (B,):
        raise ValueError("ctx_lens must be int32 [B]")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    _check_out(out, (B, Nh, Dv), q.dtype, q.device)
    st = load().attn_decode_noalloc(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), ctx_lens.data_ptr(),
                                    out.data_ptr(), B, Nh, Nkv, Dqk, Dv, max_ctx, kcache.stride(2), vcache.stride(2),
                                    float(rope_theta), float(scale or 0.0), _dtype_code(q), _stream_ptr(q.device))
    _check(st, "attn_decode_noalloc")
    return out


def decode_noalloc_max_bytes() -> int:
    return int(load().attn_decode_noalloc_max_bytes())


class kernel_events:
    """Context manager: calls made inside it by this thread record (before, after) - two
    torch.cuda.Event(enable_timing=True) - around their main attention kernel, so that
    before.elapsed_time(after) is that kernel's duration alone."""

    def __init__(self, before, after):
        self.before, self.after = before, after

    def __enter__(self):
        torch = _torch()
        for ev in (self.before, self.after):
            if not ev.cuda_event:  # torch creates the HIP event at its first record
                ev.record(torch.cuda.current_stream())
        _check(load().attn_set_kernel_events(self.before.cuda_event, self.after.cuda_event),
               "attn_set_kernel_events")
        return self

    def __exit__(self, *exc):
        load().attn_set_kernel_events(None, None)
        return False


def rope_apply_(x, *, theta: float, positions=None, interleaved: bool = False):
    """Rotate x [B, S, N, Dh] in place; positions: int32 [B, S] on the GPU or None (= s)."""
    _need_cuda(x)
    B, S, N, Dh = x.shape
    pos_ptr = None
    if positions is not None:
        _need_cuda(positions)
        if positions.numel() != B * S:
            raise ValueError("positions must hold B*S entries")
        pos_ptr = positions.data_ptr()
    st = load().rope_apply(x.data_ptr(), pos_ptr, B, S, N, Dh, float(theta), 1 if interleaved else 0,
                           _dtype_code(x), _stream_ptr(x.device))
    _check(st, "rope_apply")
    return x


def _cache_dims(t):
    """[B, max_ctx, Nkv, row] cache view -> (B, max_ctx, Nkv, row pitch in elements)."""
    if not t.is_cuda:
        raise ValueError("caches must live on the GPU")
    B_, T_, N_, _ = t.shape
    if t.stride(3) != 1 or t.stride(1) != N_ * t.stride(2) or t.stride(0) != T_ * t.stride(1):
        raise ValueError("cache must be [B, max_ctx, Nkv, row] with a dense row pitch")
    return B_, T_, N_, t.stride(2)


def prefill_cached_workspace_bytes(max_ctx: int, Dh: int, rope_theta: float) -> int:
    return int(load().attn_prefill_cached_workspace_bytes(max_ctx, Dh, float(rope_theta)))


def prefill_cached(q, kcache, vcache, q_start, *, rope_theta: float = 0.0, rope_dims: int = 0,
                   rope_interleaved: bool = False, causal: bool = True, window: int = 0, sinks: int = 0,
                   scale: float | None = None, out=None, workspace=None):
    """Chunked prefill: q [B, S, Nh, Dh] at absolute positions q_start[b] + s against the cached
    keys 0 .. q_start[b]+S-1 (already appended). kcache/vcache [B, max_ctx, Nkv, row] with the
    same row pitch; q_start int32 [B] on the GPU. window > 0: sliding window of that many keys
    plus `sinks` leading keys. Returns out [B, S, Nh, Dh]."""
    torch = _torch()
    _need_cuda(q, q_start)
    B, S, Nh, Dh = q.shape
    Bk, max_ctx, Nkv, ld = _cache_dims(kcache)
    if _cache_dims(vcache) != (Bk, max_ctx, Nkv, ld) or Bk != B:
        raise ValueError("kcache and vcache must share shape and row pitch with q's batch")
    if kcache.shape[3] < Dh or vcache.shape[3] < Dh:
        raise ValueError("cache rows shorter than the head dim")
    if q_start.dtype != torch.int32 or q_start.shape != (B,):
        raise ValueError("q_start must be int32 [B]")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    out = torch.empty_like(q) if out is None else _check_out(out, q.shape, q.dtype, q.device)
    ws_ptr, ws_bytes = _workspace(workspace, prefill_cached_workspace_bytes(max_ctx, Dh, rope_theta), q.device)
    st = load().attn_prefill_cached(q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), q_start.data_ptr(),
                                    out.data_ptr(), B, S, Nh, Nkv, Dh, max_ctx, ld, float(rope_theta), int(rope_dims),
                                    1 if rope_interleaved else 0, 1 if causal else 0, int(window), int(sinks),
                                    float(scale or 0.0),
                                    _dtype_code(q), ws_ptr, ws_bytes,
                                    _stream_ptr(q.device))
    _check(st, "attn_prefill_cached")
    return out


def kv_append(k_new, v_new, kcache, vcache, start, *, rope_theta: float = 0.0, rope_dims: int = 0,
              interleaved: bool = False):
    """Write k_new/v_new [B, S, Nkv, Dh] into the caches at rows start[b] .. start[b]+S-1,
    rotating the leading rope_dims dims of K (0: all) at those positions when rope_theta > 0.
    start: int32 [B] on the GPU."""
    torch = _torch()
    _need_cuda(k_new, v_new, start)
    B, S, Nkv, Dh = k_new.shape
    if v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must have the same shape")
    Bk, max_ctx, Nk, ldk = _cache_dims(kcache)
    Bv, max_v, Nv, ldv = _cache_dims(vcache)
    if (Bk, Nk) != (B, Nkv) or (Bv, max_v, Nv) != (B, max_ctx, Nkv):
        raise ValueError("cache shapes disagree with k_new")
    if start.dtype != torch.int32 or start.shape != (B,):
        raise ValueError("start must be int32 [B]")
    if v_new.dtype != k_new.dtype or kcache.dtype != k_new.dtype or vcache.dtype != k_new.dtype:
        raise TypeError("new rows and caches must share one dtype")
    st = load().attn_kv_append(k_new.data_ptr(), v_new.data_ptr(), kcache.data_ptr(), vcache.data_ptr(),
                               start.data_ptr(), B, S, Nkv, Dh, max_ctx, ldk, ldv, float(rope_theta), int(rope_dims),
                               1 if interleaved else 0, _dtype_code(k_new), _stream_ptr(k_new.device))
    _check(st, "attn_kv_append")
    return kcache, vcache
