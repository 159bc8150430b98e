"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function the
header declares, and rejects bad arguments before anything is launched."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _lib():
    from causal_head_attention_gqa_amd import lib
    if not os.path.exists(lib.LIB_PATH):
        pytest.fail("libattn_gfx950.so is not built (run __graft_entry__.build())")
    return lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for name in ("attn_prefill", "attn_decode", "rope_apply", "attn_prefill_workspace_bytes",
                 "attn_decode_workspace_bytes", "attn_status_str", "attn_prefill_cached",
                 "attn_prefill_cached_workspace_bytes", "attn_kv_append", "attn_prefill_mla",
                 "attn_prefill_mla_workspace_bytes"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    from causal_head_attention_gqa_amd import lib
    _lib()
    assert lib.status_str(0) == "ATTN_OK"
    assert "UNSUPPORTED" in lib.status_str(2)
    assert "unknown" in lib.status_str(99)


P = 0x10000  # a 16-byte-aligned stand-in address; these calls never reach a launch


def test_prefill_argument_errors():
    L = _lib()
    call = lambda **kw: L.attn_prefill(  # noqa: E731
        kw.get("q", P), kw.get("k", P), kw.get("v", P), kw.get("o", P), kw.get("B", 1), kw.get("S", 8),
        kw.get("Nh", 4), kw.get("Nkv", 2), kw.get("Dh", 64), kw.get("rope", 0.0), 1, 0.0, kw.get("dt", 1),
        kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(Nh=3, Nkv=2) == 1               # heads not a multiple of KV heads
    assert call(Dh=96) == 2                     # unsupported head dim
    assert call(Dh=16) == 2                     # bf16 needs 64 or 128
    assert call(dt=7) == 1                      # unknown dtype
    assert call(B=-1) == 1
    assert call(q=None) == 1                    # null pointer
    assert call(q=P + 2) == 1                   # misaligned
    assert call(rope=1e4) == 3                  # RoPE needs a workspace
    assert call(rope=1e4, ws=P, wsb=16) == 3    # too small
    assert call(rope=float("nan")) == 1
    assert call(B=0) == 0 and call(S=0) == 0    # empty: nothing to do
    # a 32-key tile of Nkv * Dh elements per row must stay addressable with 32-bit byte offsets
    assert call(Nh=1 << 20, Nkv=1 << 20) == 1


def test_decode_argument_errors():
    L = _lib()
    def call(**kw):
        return L.attn_decode(kw.get("q", P), kw.get("kc", P), kw.get("vc", P), kw.get("ctx", P), kw.get("o", P),
                             kw.get("B", 2), kw.get("Nh", 8), kw.get("Nkv", 2), kw.get("Dqk", 128), kw.get("Dv", 128),
                             kw.get("T", 100), kw.get("ldk", 128), kw.get("ldv", 128), kw.get("rope", 0.0), 0.0,
                             kw.get("dt", 1), kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(Nh=6, Nkv=4) == 1
    assert call(ldk=64) == 1                    # row pitch shorter than the row
    assert call(Dqk=96, Dv=96, ldk=96, ldv=96) == 2
    assert call(dt=0) == 2                      # fp32 decode is not built
    assert call(Nh=24, Nkv=1) == 2              # more than 16 heads per KV head only in groups of 16
    assert call(Dqk=576, Dv=512, Nkv=1, Nh=128, ldk=576, ldv=576, vc=P + 4096) == 2  # MLA needs V aliasing K
    assert call(Dqk=576, Dv=512, Nkv=1, Nh=128, ldk=576, ldv=576, rope=1e4) == 3  # decoupled RoPE: supported
    assert call() == 3                          # no workspace
    assert call(ws=P, wsb=8) == 3
    assert call(ctx=None) == 1
    assert call(B=0) == 0


def test_rope_argument_errors():
    L = _lib()
    assert L.rope_apply(P, None, 1, 4, 2, 63, 1e4, 0, 1, None) == 1   # odd head dim
    assert L.rope_apply(P, None, 1, 4, 2, 64, 0.0, 0, 1, None) == 1   # theta must be > 0
    assert L.rope_apply(P, None, 1, 4, 2, 2048, 1e4, 0, 1, None) == 2
    assert L.rope_apply(P + 1, None, 1, 4, 2, 64, 1e4, 0, 1, None) == 1
    assert L.rope_apply(P, None, 0, 4, 2, 64, 1e4, 0, 1, None) == 0


def test_workspace_queries():
    from causal_head_attention_gqa_amd import lib
    _lib()
    # bf16: 512 bytes for the work lists' counters (8, 64 bytes apart), optional; fp32 has none
    assert lib.prefill_workspace_bytes(4, 8192, 8, 128, 0.0, 1) == 512
    assert lib.prefill_workspace_bytes(4, 8192, 8, 64, 0.0, 0) == 0
    # RoPE: fp32 (cos, sin) table [S, Dh/2] plus rotated keys (required), then the counters
    assert lib.prefill_workspace_bytes(4, 8192, 8, 128, 5e5, 1) == 8192 * 64 * 8 + 4 * 8192 * 8 * 128 * 2 + 512
    ws = lib.decode_workspace_bytes(64, 32, 8, 128, 128, 8192, 1)
    assert ws > 0 and ws % 256 == 0
    # MLA: split partials (bf16 rows + fp32 max/sum) for 8 chunks of 512 tokens at B = 32 ...
    assert lib.decode_workspace_bytes(32, 128, 1, 576, 512, 4096, 1) == 32 * 128 * 8 * 512 * 2 + 32 * 128 * 8 * 2 * 4
    # ... none once every sequence is one chunk (256 sequences fill the chip)
    assert lib.decode_workspace_bytes(256, 128, 1, 576, 512, 64, 1) == 0


def test_prefill_cached_argument_errors():
    L = _lib()
    def call(**kw):
        return L.attn_prefill_cached(kw.get("q", P), kw.get("kc", P), kw.get("vc", P), kw.get("st", P),
                                     kw.get("o", P), kw.get("B", 2), kw.get("S", 16), kw.get("Nh", 8),
                                     kw.get("Nkv", 2), kw.get("Dh", 128), kw.get("T", 100), kw.get("ld", 128),
                                     kw.get("rope", 0.0), kw.get("rdims", 0), 0, kw.get("causal", 1), kw.get("win", 0),
                                     kw.get("sinks", 0),
                                     0.0, kw.get("dt", 1), kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(S=101) == 1                     # chunk longer than the cache
    assert call(ld=64) == 1                     # row pitch shorter than the head dim
    assert call(ld=132) == 1                    # rows not 16-byte aligned
    assert call(Nh=6, Nkv=4) == 1
    assert call(Dh=96, ld=96) == 2
    assert call(dt=0) == 2                      # bf16 only
    assert call(st=None) == 1
    assert call(rope=5e5) == 3                  # the angle table needs a workspace
    assert call(win=-1) == 1
    assert call(win=64, causal=0) == 1          # a window needs the causal mask
    assert call(sinks=4) == 1                   # sinks only with a window
    assert call(rdims=256) == 1                 # rotary span longer than the head
    assert call(rdims=48) == 2                  # q is rotated in 32-dim groups
    assert call(B=0) == 0 and call(S=0) == 0


def test_kv_append_argument_errors():
    L = _lib()
    def call(**kw):
        return L.attn_kv_append(kw.get("k", P), kw.get("v", P), kw.get("kc", P), kw.get("vc", P), kw.get("st", P),
                                kw.get("B", 2), kw.get("S", 16), kw.get("Nkv", 2), kw.get("Dh", 128),
                                kw.get("T", 100), kw.get("ldk", 128), kw.get("ldv", 128), kw.get("rope", 1e4),
                                kw.get("rdims", 0), 0, kw.get("dt", 1), None)
    assert call(S=101) == 1
    assert call(ldv=100) == 1
    assert call(Dh=68, ldk=72, ldv=72) == 2     # head dim not a multiple of 8
    assert call(rdims=33) == 1                  # odd rotary span
    assert call(dt=0) == 2
    assert call(st=None) == 1
    assert call(rope=float("inf")) == 1
    assert call(B=0) == 0


def test_prefill_cached_workspace_query():
    from causal_head_attention_gqa_amd import lib
    _lib()
    # the angle table (required with RoPE), then 512 bytes of optional work-list counters
    assert lib.prefill_cached_workspace_bytes(8192, 128, 0.0) == 512
    assert lib.prefill_cached_workspace_bytes(8192, 128, 5e5) == 8192 * 64 * 8 + 512


def test_prefill_mla_argument_errors():
    L = _lib()
    def call(**kw):
        return L.attn_prefill_mla(kw.get("q", P), kw.get("k", P), kw.get("v", P), kw.get("o", P), kw.get("B", 2),
                                  kw.get("S", 16), kw.get("Nh", 8), kw.get("Nkv", 8), kw.get("rope", 0.0), 1,
                                  kw.get("scale", 0.0), kw.get("ws", None), kw.get("wsb", 0), None)
    assert call(Nh=6, Nkv=4) == 1
    assert call(Nkv=0) == 1
    assert call(v=None) == 1
    assert call(o=P + 8) == 1                   # misaligned
    assert call(rope=1e4) == 3                  # k^R rotation needs a workspace
    assert call(rope=1e4, ws=P, wsb=64) == 3
    assert call(rope=float("nan")) == 1
    assert call(scale=float("inf")) == 1
    assert call(B=0) == 0 and call(S=0) == 0
    # (valid arguments would launch: never with these stand-in addresses)


def test_prefill_mla_workspace_query():
    from causal_head_attention_gqa_amd import lib
    _lib()
    assert lib.prefill_mla_workspace_bytes(1, 4096, 128, 0.0) == 512  # the optional work-list counters
    # fp32 (cos, sin) table [S, 32] plus keys with the rotated k^R block
    assert lib.prefill_mla_workspace_bytes(1, 4096, 128, 1e4) == 4096 * 32 * 8 + 4096 * 128 * 192 * 2 + 512


class _FakeTensor:
    """Just enough of a device tensor for the binding's checks of caller-supplied buffers."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True, cuda=True):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = cuda
        self._c = contiguous

    def is_contiguous(self):
        return self._c


def test_binding_rejects_mismatched_out_buffers():
    import torch
    from causal_head_attention_gqa_amd import lib
    dev = torch.device("cuda:0")
    good = _FakeTensor((2, 8, 4, 64), torch.bfloat16)
    assert lib._check_out(good, (2, 8, 4, 64), torch.bfloat16, dev) is good
    with pytest.raises(ValueError):
        lib._check_out(_FakeTensor((2, 8, 4, 32), torch.bfloat16), (2, 8, 4, 64), torch.bfloat16, dev)  # too small
    with pytest.raises(TypeError):
        lib._check_out(_FakeTensor((2, 8, 4, 64), torch.float32), (2, 8, 4, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError):
        lib._check_out(_FakeTensor((2, 8, 4, 64), torch.bfloat16, contiguous=False), (2, 8, 4, 64),
                       torch.bfloat16, dev)
    with pytest.raises(ValueError):
        lib._check_out(_FakeTensor((2, 8, 4, 64), torch.bfloat16, device="cpu", cuda=False), (2, 8, 4, 64),
                       torch.bfloat16, dev)
    with pytest.raises(ValueError):
        lib._check_out(_FakeTensor((2, 8, 4, 64), torch.bfloat16, device="cuda:1"), (2, 8, 4, 64),
                       torch.bfloat16, dev)


def test_binding_rejects_foreign_workspaces():
    import torch
    from causal_head_attention_gqa_amd import lib
    dev = torch.device("cuda:0")
    with pytest.raises(ValueError):
        lib._workspace(_FakeTensor((64,), torch.uint8, device="cpu", cuda=False), 64, dev)
    with pytest.raises(ValueError):
        lib._workspace(_FakeTensor((64,), torch.uint8, contiguous=False), 64, dev)
    assert lib._workspace(None, 0, dev) == (None, 0)
