// C ABI of the library: argument validation on the host, workspace layout, kernel dispatch.
// Nothing is launched unless every argument has been checked; no exception crosses the ABI.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "kernels.hpp"

using namespace attn;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t esize(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

bool prefill_supported(int dtype, int Dh) {
  if (dtype == ATTN_BF16) return Dh == 64 || Dh == 128;
  if (dtype == ATTN_F32) return Dh == 16 || Dh == 32 || Dh == 64;
  return false;
}

// Split-KV plan shared by the workspace query and the call.
struct DecodePlan {
  int chunk = 0, nsplit = 0;
  bool mla = false;
};

bool is_mla_shape(int Nkv, int Dqk, int Dv) { return Dqk == 576 && Dv == 512 && Nkv == 1; }

DecodePlan decode_plan(int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx) {
  DecodePlan p;
  p.mla = is_mla_shape(Nkv, Dqk, Dv);
  if (max_ctx <= 0 || B <= 0) return p;
  if (p.mla) {
    // one work-group per (sequence, head group, chunk); one such work-group fills a CU (128- and
    // 64-head groups: 153 and 160 KiB of LDS, one wave per SIMD), so aim for about 256 work-groups
    const long long groups = (long long)B * (Nh / mla_heads_per_group(Nh));
    const int tiles = (max_ctx + 31) / 32;
    long long want = (256 + groups - 1) / groups;  // about one work-group per CU
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    const int per = (int)((max_ctx + want - 1) / want);
    p.chunk = (per + 31) / 32 * 32;
  } else {
    // work-groups of (sequence, KV head, up to 16 query heads, chunk); 1024-token chunks unless
    // that leaves fewer than ~1024 work-groups
    const int G = Nh / Nkv;
    const long long groups = (long long)B * Nkv * (G < 16 ? 1 : G / 16);
    p.chunk = 1024;
    while (p.chunk > 64 && groups * ((max_ctx + p.chunk - 1) / p.chunk) < 1024) p.chunk /= 2;
  }
  p.nsplit = (max_ctx + p.chunk - 1) / p.chunk;
  return p;
}

hipError_t g_last_hip = hipSuccess;

// Scratch of attn_decode_noalloc: the split-KV partials live in this file-scope device array
// instead of a caller workspace. Every GPU the library runs on holds its own copy from the
// first use until the process ends. On the host, `scratch` names a host-side stand-in, not device
// memory: host code uses only the per-device address that hipGetSymbolAddress returns.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) static unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ATTN_OK;
  g_last_hip = e;
  return ATTN_ERR_HIP;
}

// Profiling hook (attn_set_kernel_events): events recorded right before and right after the main
// attention kernel of each call made by this host thread.
thread_local hipEvent_t t_ev_before = nullptr;
thread_local hipEvent_t t_ev_after = nullptr;

// Launches `fn` on st between the caller's profiling events, when set.
template <typename F>
hipError_t timed_launch(hipStream_t st, F&& fn) {
  if (t_ev_before) {
    const hipError_t e = hipEventRecord(t_ev_before, st);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = fn();
  if (e != hipSuccess || !t_ev_after) return e;
  return hipEventRecord(t_ev_after, st);
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK:
      return "ATTN_OK";
    case ATTN_ERR_INVALID:
      return "ATTN_ERR_INVALID: invalid argument";
    case ATTN_ERR_UNSUPPORTED:
      return "ATTN_ERR_UNSUPPORTED: shape or dtype outside the built kernel set";
    case ATTN_ERR_WORKSPACE:
      return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_HIP:
      return "ATTN_ERR_HIP: HIP runtime error";
    default:
      return "unknown attn status";
  }
}

// Workspace bytes attn_prefill cannot run without: the RoPE angle table and the rotated K copy.
size_t prefill_rope_bytes(int B, int S, int Nkv, int Dh, float rope_theta, int dtype) {
  if (!(rope_theta > 0.f) || B <= 0 || S <= 0 || Nkv <= 0 || Dh <= 0) return 0;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
  const size_t table = align_up((size_t)S * (size_t)(Dh / 2) * sizeof(float2));
  const size_t krot = align_up((size_t)B * (size_t)S * (size_t)Nkv * (size_t)Dh * esize(dtype));
  return table + krot;
}

size_t attn_prefill_workspace_bytes(int B, int S, int Nkv, int Dh, float rope_theta, int dtype) {
  if (B <= 0 || S <= 0 || Nkv <= 0 || Dh <= 0) return 0;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return 0;
  // bf16: the work lists' counters after the RoPE part
  return prefill_rope_bytes(B, S, Nkv, Dh, rope_theta, dtype) + (dtype == ATTN_BF16 ? kPrefillQueueBytes : 0);
}

int attn_prefill(const void* q, const void* k, const void* v, void* out, int B, int S, int Nh, int Nkv, int Dh,
                 float rope_theta, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (B < 0 || S < 0 || Nh <= 0 || Nkv <= 0 || Dh <= 0) return ATTN_ERR_INVALID;
  if (Nh % Nkv != 0) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (!std::isfinite(rope_theta) || !std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (!prefill_supported(dtype, Dh)) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * S * Nh > (1LL << 40)) return ATTN_ERR_INVALID;
  // the bf16 kernel addresses a 32-key tile with 32-bit per-lane byte offsets (32 rows of Nkv*Dh)
  if ((long long)Nkv * Dh * 32 * (long long)esize(dtype) > 0x7fffffffLL) return ATTN_ERR_INVALID;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_INVALID;
  const bool rope = rope_theta > 0.f;
  // the RoPE part is required; the counters after it are optional (without them, or without any
  // workspace when there is no RoPE, each work-group's item follows from its id)
  const size_t need = prefill_rope_bytes(B, S, Nkv, Dh, rope_theta, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_ERR_WORKSPACE;
  const bool lists = dtype == ATTN_BF16 && workspace != nullptr && aligned16(workspace) &&
                     workspace_bytes >= need + kPrefillQueueBytes;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)Dh);
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.table = nullptr;
  a.B = B;
  a.S = S;
  a.Nh = Nh;
  a.Nkv = Nkv;
  a.D = Dh;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = causal ? 1 : 0;
  a.Dv = Dh;
  a.kv_tok = (long long)Nkv * Dh;
  a.kv_batch = (long long)S * Nkv * Dh;
  a.kv_head = Dh;
  a.v_tok = a.kv_tok;
  a.v_batch = a.kv_batch;
  a.v_head = a.kv_head;
  a.q_start = nullptr;
  a.max_keys = S;
  a.window = 0;
  a.sinks = 0;
  a.rope_dims = Dh;
  a.rope_inter = 0;
  a.queue = lists ? reinterpret_cast<unsigned int*>(static_cast<char*>(workspace) + need) : nullptr;

  if (rope) {
    float2* table = static_cast<float2*>(workspace);
    void* krot = static_cast<char*>(workspace) + align_up((size_t)S * (size_t)(Dh / 2) * sizeof(float2));
    hipError_t e;
    if (dtype == ATTN_BF16) {
      e = launch_rope_table_rotate_bf16(static_cast<const bf16_t*>(k), static_cast<bf16_t*>(krot), table, B, S, Nkv,
                                        Dh, (double)rope_theta, st, a.queue, &a.queue_zeroed);
    } else {
      e = launch_rope_table(table, S, Dh, (double)rope_theta, st);
      if (e == hipSuccess)
        e = launch_rope_rotate_table<float>(static_cast<const float*>(k), static_cast<float*>(krot), table,
                                            (long long)B * S * Nkv, S, Nkv, Dh, st);
    }
    if (e != hipSuccess) return hip_status(e);
    a.table = table;
    a.k = krot;
  }
  return hip_status(timed_launch(st, [&] { return dtype == ATTN_BF16 ? launch_prefill_bf16(a, st)
                                                                     : launch_prefill_f32(a, st); }));
}

// Required part of the MLA prefill's workspace: the k^R angle table and the keys with their rotated k^R.
size_t prefill_mla_rope_bytes(int B, int S, int Nkv, float rope_theta) {
  if (!(rope_theta > 0.f) || B <= 0 || S <= 0 || Nkv <= 0) return 0;
  return align_up((size_t)S * 32 * sizeof(float2)) + align_up((size_t)B * S * Nkv * 192 * 2);
}

size_t attn_prefill_mla_workspace_bytes(int B, int S, int Nkv, float rope_theta) {
  if (B <= 0 || S <= 0 || Nkv <= 0) return 0;
  return prefill_mla_rope_bytes(B, S, Nkv, rope_theta) + kPrefillQueueBytes;  // then the work lists' counters
}

int attn_prefill_mla(const void* q, const void* k, const void* v, void* out, int B, int S, int Nh, int Nkv,
                     float rope_theta, int causal, float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (B < 0 || S < 0 || Nh <= 0 || Nkv <= 0 || Nh % Nkv != 0) return ATTN_ERR_INVALID;
  if (!std::isfinite(rope_theta) || !std::isfinite(scale)) return ATTN_ERR_INVALID;
  if ((long long)B * S * Nh > (1LL << 40) || (long long)Nkv * 192 * 32 > 0x7fffffffLL) return ATTN_ERR_INVALID;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_INVALID;
  // the RoPE part is required, the work lists' counters after it optional
  const size_t need = prefill_mla_rope_bytes(B, S, Nkv, rope_theta);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_ERR_WORKSPACE;
  const bool lists = workspace != nullptr && aligned16(workspace) && workspace_bytes >= need + kPrefillQueueBytes;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt(192.0);
  PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.table = nullptr;
  a.B = B;
  a.S = S;
  a.Nh = Nh;
  a.Nkv = Nkv;
  a.D = 192;
  a.Dv = 128;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = causal ? 1 : 0;
  a.kv_tok = (long long)Nkv * 192;
  a.kv_batch = (long long)S * Nkv * 192;
  a.kv_head = 192;
  a.v_tok = (long long)Nkv * 128;
  a.v_batch = (long long)S * Nkv * 128;
  a.v_head = 128;
  a.q_start = nullptr;
  a.max_keys = S;
  a.window = 0;
  a.sinks = 0;
  a.rope_dims = 64;
  a.rope_inter = 0;
  a.queue = lists ? reinterpret_cast<unsigned int*>(static_cast<char*>(workspace) + need) : nullptr;
  if (rope_theta > 0.f) {
    float2* table = static_cast<float2*>(workspace);
    void* krot = static_cast<char*>(workspace) + align_up((size_t)S * 32 * sizeof(float2));
    hipError_t e = launch_rope_table(table, S, 64, (double)rope_theta, st);
    if (e != hipSuccess) return hip_status(e);
    e = launch_rope_span_table(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(krot), table,
                               (long long)B * S * Nkv, S, Nkv, 192, 128, 64, st);
    if (e != hipSuccess) return hip_status(e);
    a.table = table;
    a.k = krot;
  }
  return hip_status(timed_launch(st, [&] { return launch_prefill_bf16(a, st); }));
}

// Required part of the chunked prefill's workspace: the angle table of the query positions.
size_t prefill_cached_rope_bytes(int max_ctx, int Dh, float rope_theta) {
  if (!(rope_theta > 0.f) || max_ctx <= 0 || Dh <= 0) return 0;
  return align_up((size_t)max_ctx * (size_t)(Dh / 2) * sizeof(float2));
}

size_t attn_prefill_cached_workspace_bytes(int max_ctx, int Dh, float rope_theta) {
  if (max_ctx <= 0 || Dh <= 0) return 0;
  return prefill_cached_rope_bytes(max_ctx, Dh, rope_theta) + kPrefillQueueBytes;  // then the lists' counters
}

int attn_prefill_cached(const void* q, const void* kcache, const void* vcache, const int32_t* q_start, void* out,
                        int B, int S, int Nh, int Nkv, int Dh, int max_ctx, long long ld, float rope_theta,
                        int rope_dims, int rope_interleaved, int causal, int window, int sinks, float scale,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || S < 0 || Nh <= 0 || Nkv <= 0 || Dh <= 0 || max_ctx <= 0) return ATTN_ERR_INVALID;
  if (window < 0 || sinks < 0 || (window > 0 && !causal) || (window == 0 && sinks > 0)) return ATTN_ERR_INVALID;
  if (rope_dims == 0) rope_dims = Dh;
  if (rope_dims < 0 || rope_dims > Dh) return ATTN_ERR_INVALID;
  if (Nh % Nkv != 0 || S > max_ctx || ld < Dh || ld % 8 != 0) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (!std::isfinite(rope_theta) || !std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 || (Dh != 64 && Dh != 128)) return ATTN_ERR_UNSUPPORTED;
  if (rope_dims % 32 != 0) return ATTN_ERR_UNSUPPORTED;  // q is rotated in 32-dim register groups
  if ((long long)B * max_ctx * Nkv * ld > (1LL << 40) || (long long)Nkv * ld * 32 > 0x7fffffffLL)
    return ATTN_ERR_INVALID;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!q || !kcache || !vcache || !q_start || !out) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out)) return ATTN_ERR_INVALID;
  // the angle table is required, the work lists' counters after it optional (bf16)
  const size_t need = prefill_cached_rope_bytes(max_ctx, Dh, rope_theta);
  const bool lists = dtype == ATTN_BF16 && workspace != nullptr && aligned16(workspace) &&
                     workspace_bytes >= need + kPrefillQueueBytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
    return ATTN_ERR_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)Dh);
  PrefillArgs a{};
  a.q = q;
  a.k = kcache;
  a.v = vcache;
  a.out = out;
  a.table = nullptr;
  a.B = B;
  a.S = S;
  a.Nh = Nh;
  a.Nkv = Nkv;
  a.D = Dh;
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.causal = causal ? 1 : 0;
  a.Dv = Dh;
  a.kv_tok = (long long)Nkv * ld;
  a.kv_batch = (long long)max_ctx * Nkv * ld;
  a.kv_head = (int)ld;
  a.v_tok = a.kv_tok;
  a.v_batch = a.kv_batch;
  a.v_head = a.kv_head;
  a.q_start = q_start;
  a.max_keys = max_ctx;
  a.window = window;
  a.sinks = sinks;
  a.rope_dims = rope_dims;
  a.rope_inter = rope_interleaved ? 1 : 0;
  a.queue = lists ? reinterpret_cast<unsigned int*>(static_cast<char*>(workspace) + need) : nullptr;
  if (rope_theta > 0.f) {
    float2* table = static_cast<float2*>(workspace);
    const hipError_t e = launch_rope_table(table, max_ctx, rope_dims, (double)rope_theta, st);
    if (e != hipSuccess) return hip_status(e);
    a.table = table;
  }
  return hip_status(timed_launch(st, [&] { return launch_prefill_bf16(a, st); }));
}

int attn_kv_append(const void* k_new, const void* v_new, void* kcache, void* vcache, const int32_t* start, int B,
                   int S, int Nkv, int Dh, int max_ctx, long long ldk, long long ldv, float rope_theta,
                   int rope_dims, int interleaved, int dtype, void* stream) {
  if (B < 0 || S < 0 || Nkv <= 0 || Dh <= 0 || max_ctx <= 0 || S > max_ctx) return ATTN_ERR_INVALID;
  if (rope_dims == 0) rope_dims = Dh;
  if (rope_dims < 0 || rope_dims > Dh || rope_dims % 2 != 0) return ATTN_ERR_INVALID;
  if (ldk < Dh || ldv < Dh) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (!std::isfinite(rope_theta)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 || Dh % 8 != 0 || Dh > 1024) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * max_ctx * Nkv * (ldk > ldv ? ldk : ldv) > (1LL << 40)) return ATTN_ERR_INVALID;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!k_new || !v_new || !kcache || !vcache || !start) return ATTN_ERR_INVALID;
  return hip_status(launch_kv_append(static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                     static_cast<uint16_t*>(kcache), static_cast<uint16_t*>(vcache), start, B, S,
                                     Nkv, Dh, max_ctx, ldk, ldv, (double)rope_theta, rope_dims, interleaved,
                                     static_cast<hipStream_t>(stream)));
}

size_t attn_decode_workspace_bytes(int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx, int dtype) {
  if (B <= 0 || Nh <= 0 || Nkv <= 0 || Dv <= 0 || max_ctx <= 0 || dtype != ATTN_BF16) return 0;
  if (Nh % Nkv != 0) return 0;
  const DecodePlan p = decode_plan(B, Nh, Nkv, Dqk, Dv, max_ctx);
  if (p.mla && p.nsplit == 1) return 0;  // one chunk per sequence: the kernel writes the output itself
  const size_t slots = (size_t)B * (size_t)Nh * (size_t)p.nsplit;
  return align_up(slots * (size_t)Dv * sizeof(uint16_t)) + align_up(slots * 2 * sizeof(float));
}

int attn_decode(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out, int B,
                int Nh, int Nkv, int Dqk, int Dv, int max_ctx, long long ldk, long long ldv, float rope_theta,
                float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || Nh <= 0 || Nkv <= 0 || Dqk <= 0 || Dv <= 0 || max_ctx <= 0) return ATTN_ERR_INVALID;
  if (Nh % Nkv != 0 || ldk < Dqk || ldv < Dv) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (!std::isfinite(rope_theta) || !std::isfinite(scale)) return ATTN_ERR_INVALID;
  if (ldk % 8 != 0 || ldv % 8 != 0) return ATTN_ERR_INVALID;  // 16-byte aligned rows
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  const bool mla = is_mla_shape(Nkv, Dqk, Dv);
  if (mla) {
    if (vcache != kcache || ldv != ldk || Nh % 16 != 0) return ATTN_ERR_UNSUPPORTED;
    if (ldk * 64 > 0x7fffffffLL) return ATTN_ERR_INVALID;  // 32-bit byte offsets within a 32-row tile
  } else {
    if (Dqk != Dv || (Dqk != 64 && Dqk != 128)) return ATTN_ERR_UNSUPPORTED;
    if (Nh / Nkv > 16 && (Nh / Nkv) % 16 != 0) return ATTN_ERR_UNSUPPORTED;  // heads go in groups of 16
  }
  if (B == 0) return ATTN_OK;
  if (!q || !kcache || !vcache || !ctx_lens || !out) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(ctx_lens) & 3u))
    return ATTN_ERR_INVALID;
  const size_t need = attn_decode_workspace_bytes(B, Nh, Nkv, Dqk, Dv, max_ctx, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))) return ATTN_ERR_WORKSPACE;

  const DecodePlan p = decode_plan(B, Nh, Nkv, Dqk, Dv, max_ctx);
  const size_t slots = need > 0 ? (size_t)B * (size_t)Nh * (size_t)p.nsplit : 0;
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kcache);
  a.vc = static_cast<const uint16_t*>(vcache);
  a.ctx_lens = ctx_lens;
  a.out = static_cast<uint16_t*>(out);
  // no partials when the workspace is not needed (the kernels then never touch these pointers)
  a.part_o = need > 0 ? static_cast<uint16_t*>(workspace) : nullptr;
  a.part_ml = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(slots * (size_t)Dv * sizeof(uint16_t)))
                       : nullptr;
  a.B = B;
  a.Nh = Nh;
  a.Nkv = Nkv;
  a.Dqk = Dqk;
  a.Dv = Dv;
  a.max_ctx = max_ctx;
  a.ldk = ldk;
  a.ldv = ldv;
  const double sc = scale > 0.f ? (double)scale : 1.0 / std::sqrt((double)Dqk);
  a.scale_log2 = (float)(sc * 1.4426950408889634);
  a.rope_theta = rope_theta > 0.f ? (double)rope_theta : 0.0;
  a.chunk = p.chunk;
  a.nsplit = p.nsplit;

  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed_launch(st, [&] { return mla ? launch_decode_mla(a, st) : launch_decode_gqa(a, st); });
  if (e != hipSuccess) return hip_status(e);
  if (mla && p.nsplit == 1) return ATTN_OK;  // a single chunk already wrote the output
  return hip_status(launch_decode_reduce(a, st));
}

size_t attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int attn_set_kernel_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return ATTN_ERR_INVALID;
  t_ev_before = static_cast<hipEvent_t>(before);
  t_ev_after = static_cast<hipEvent_t>(after);
  return ATTN_OK;
}

int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* ctx_lens, void* out,
                        int B, int Nh, int Nkv, int Dqk, int Dv, int max_ctx, long long ldk, long long ldv,
                        float rope_theta, float scale, int dtype, void* stream) {
  // the split partials must fit the static scratch; anything else is validated by attn_decode
  const size_t need = attn_decode_workspace_bytes(B, Nh, Nkv, Dqk, Dv, max_ctx, dtype);
  if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;
  if (B <= 0) {  // nothing to launch: attn_decode validates and returns without touching the scratch
    return attn_decode(q, kcache, vcache, ctx_lens, out, B, Nh, Nkv, Dqk, Dv, max_ctx, ldk, ldv, rope_theta, scale,
                       dtype, nullptr, 0, stream);
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  return attn_decode(q, kcache, vcache, ctx_lens, out, B, Nh, Nkv, Dqk, Dv, max_ctx, ldk, ldv, rope_theta, scale,
                     dtype, ws, kScratchBytes, stream);
}

int rope_apply(void* x, const int32_t* positions, int B, int S, int N, int Dh, float theta, int interleaved,
               int dtype, void* stream) {
  if (B < 0 || S < 0 || N <= 0 || Dh <= 0 || Dh % 2 != 0) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (!std::isfinite(theta) || !(theta > 0.f)) return ATTN_ERR_INVALID;
  if (Dh > 1024) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || S == 0) return ATTN_OK;
  if (!x) return ATTN_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(x) & (esize(dtype) - 1)) || (reinterpret_cast<uintptr_t>(positions) & 3u))
    return ATTN_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const long long rows = (long long)B * S * N;
  const hipError_t e =
      dtype == ATTN_BF16
          ? launch_rope_apply<bf16_t>(static_cast<bf16_t*>(x), positions, rows, S, N, Dh, (double)theta,
                                      interleaved ? 1 : 0, st)
          : launch_rope_apply<float>(static_cast<float*>(x), positions, rows, S, N, Dh, (double)theta,
                                     interleaved ? 1 : 0, st);
  return hip_status(e);
}

}  // extern "C"
