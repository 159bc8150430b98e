// Launchers of the gfx950 kernels, called by the C ABI in api.hip after argument validation.
// Every launcher only enqueues work on `st` and returns hipGetLastError().
#pragma once

#include "common.hpp"

namespace attn {

// bf16 storage element (bit pattern); arithmetic is always done in fp32.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return bf16_t{f32_to_bf16(x)}; }

// ---- RoPE (rope.hip) ----
hipError_t launch_rope_table(float2* table, int S, int D, double theta, hipStream_t st);
// The table and the bf16 rotation of K [B, S, N, D] (positions 0 .. S-1) in one launch.
// zero: 128 words the one-launch form also zeroes (the prefill's work-list counters, which then
// need no launch of their own), or nullptr; *zeroed tells whether it did.
hipError_t launch_rope_table_rotate_bf16(const bf16_t* src, bf16_t* dst, float2* table, int B, int S, int N, int D,
                                         double theta, hipStream_t st, unsigned int* zero = nullptr,
                                         bool* zeroed = nullptr);
template <typename T>
hipError_t launch_rope_rotate_table(const T* src, T* dst, const float2* table, long long rows, int S, int N,
                                    int D, hipStream_t st);
template <typename T>
hipError_t launch_rope_apply(T* x, const int* positions, long long rows, int S, int N, int D, double theta,
                             int interleaved, hipStream_t st);
hipError_t launch_rope_span_table(const uint16_t* src, uint16_t* dst, const float2* table, long long rows, int S,
                                  int N, int D, int roff, int Dr, hipStream_t st);
hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* kc, uint16_t* vc,
                            const int* start, int B, int S, int Nkv, int D, int max_ctx, long long ldk, long long ldv,
                            double theta, int Dr, int interleaved, hipStream_t st);

// ---- Prefill (prefill_f32.hip, prefill_bf16.hip) ----
struct PrefillArgs {
  const void* q;
  const void* k;  // rotated copy when table != nullptr
  const void* v;
  void* out;
  const float2* table;  // [S][D/2] (cos, sin) or nullptr: q used as given
  int B, S, Nh, Nkv, D;
  int Dv;            // head dim of v and out (bf16 path; D is the q/k head dim)
  float scale_log2;  // softmax scale * log2(e)
  int causal;
  // K/V addressing (bf16 path): element (b, t, g, d) of K at b*kv_batch + t*kv_tok + g*kv_head + d,
  // of V at b*v_batch + t*v_tok + g*v_head + d
  long long kv_tok, kv_batch;
  int kv_head;
  long long v_tok, v_batch;
  int v_head;
  const int* q_start;  // device [B]: absolute position of query 0 of each sequence, or nullptr (0)
  int max_keys;        // keys available per sequence (q_start[b] + S is clamped to it)
  int window;          // > 0: a query at position p sees keys p-window+1 .. p only (plus the sinks)
  int sinks;           // with a window: keys 0 .. sinks-1 stay visible to every later query
  int rope_dims;       // with a table: rotary span = the leading rope_dims dims (multiple of 32)
  int rope_inter;      // with a table: adjacent pairs (2j, 2j+1) instead of (i, i + rope_dims/2)
  // bf16 path: kPrefillQueueBytes of device memory for the work lists' counters (zeroed at the
  // launch), or nullptr: each work-group's item follows from its id
  unsigned int* queue;
  bool queue_zeroed;  // the counters were zeroed by an earlier launch on the stream (the RoPE pre-pass)
};
constexpr size_t kPrefillQueueBytes = 512;  // 8 counters, 64 bytes apart
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st);

// ---- Decode (decode.hip, decode_mla.hip) ----
struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int* ctx_lens;
  uint16_t* out;
  uint16_t* part_o;  // [B][nsplit][Nh][Dv] bf16: the chunk's output normalised by its own sum
  float* part_ml;    // [B][nsplit][Nh][2]  fp32 (reference max in log2 units, sum)
  int B, Nh, Nkv, Dqk, Dv, max_ctx;
  long long ldk, ldv;
  float scale_log2;
  double rope_theta;  // <= 0: none
  int chunk, nsplit;
};
// Partial slot of (sequence b, query head h, chunk s): chunk-major within a sequence, so that the
// heads of one chunk are adjacent and a work-group's partials form one contiguous block.
__device__ __forceinline__ long long part_slot(const DecodeArgs& a, int b, int h, int s) {
  return ((long long)b * a.nsplit + s) * a.Nh + h;
}
hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st);
int mla_waves_per_group(int Nh);  // waves (16 heads each) per MLA work-group
int mla_heads_per_group(int Nh);  // query heads per MLA work-group
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st);

}  // namespace attn
