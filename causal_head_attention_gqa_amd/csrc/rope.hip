// RoPE on gfx950: angle table, table-driven rotation (prefill pre-pass for K) and the standalone
// in-place rotation with arbitrary positions.
//
// Frequencies theta_i = base^(-2i/D), i = 0 .. D/2-1 ("2.7 Transformer Decoder Block完整解析" §4,
// "Transformer 架构快速入门" §8.2); angle = position * theta_i, evaluated in fp64 so that large
// positions keep full fp32 accuracy after the single rounding of cos/sin. Half-split pairs
// (i, i + D/2) follow the first page's apply_rope; adjacent pairs (2i, 2i+1) follow
// "Transformer 架构快速入门" §8.3. Only Q and K are rotated (same page, §8.5).
#include <type_traits>

#include "kernels.hpp"

namespace attn {

// (cos, sin) of position * theta_i: fp64 angle, one rounding to fp32. The angle table and the
// fused cache append both use this, so a key rotated by either carries identical bits.
__device__ __forceinline__ float2 rope_cs(int pos, int i, double neg2_log2theta_over_d) {
  const double inv_freq = exp2(neg2_log2theta_over_d * (double)i);
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  return make_float2((float)c, (float)s);
}

// Rotation of the pair (a, b) by (cos, sin) in fp32 with fixed fused-multiply-add rounding.
__device__ __forceinline__ float2 rope_rot(float a, float b, float2 cs) {
  return make_float2(fmaf(a, cs.x, -(b * cs.y)), fmaf(a, cs.y, b * cs.x));
}

// table[pos * half + i] = (cos(pos * theta_i), sin(pos * theta_i)), fp64 angle, fp32 result.
__global__ void rope_table_kernel(float2* __restrict__ table, int S, int half, double neg2_log2theta_over_d) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)S * half) return;
  table[idx] = rope_cs((int)(idx / half), (int)(idx % half), neg2_log2theta_over_d);
}

// Rotates half-split pairs of src [rows, D] (row r has position (r / N) % S) into dst with the
// table. Each thread owns 8 consecutive pair indices of one row: two 8-element vectors.
template <typename T>
__global__ void rope_rotate_table_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                         const float2* __restrict__ table, long long rows, int S, int N,
                                         int D) {
  const int groups = D / 16;  // 8 pairs per thread
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * groups) return;
  const long long row = idx / groups;
  const int i0 = (int)(idx % groups) * 8;
  const int pos = (int)((row / N) % S);
  const T* x = src + row * D;
  T* y = dst + row * D;
  const float2* tb = table + (long long)pos * (D / 2) + i0;
  float a[8], b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = to_f32(x[i0 + e]);
    b[e] = to_f32(x[i0 + D / 2 + e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float2 r = rope_rot(a[e], b[e], tb[e]);
    y[i0 + e] = from_f32<T>(r.x);
    y[i0 + D / 2 + e] = from_f32<T>(r.y);
  }
}

// bf16 form of the same rotation, for K of shape [B, S, N, D]: a thread owns 8 consecutive pair
// indices of the rows (b, s, g) for every b, so its 8 (cos, sin) entries are read once and used B
// times, and it moves whole 16-byte vectors (a wave covers the N*D contiguous elements of one
// (b, s) for N*D/16 = 64 threads, e.g. N = 8, D = 128).
__global__ void rope_rotate_table_bf16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                              const float2* __restrict__ table, int B, int S, int N, int D) {
  const int groups = D / 16;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)S * N * groups) return;
  const int i0 = (int)(idx % groups) * 8;
  const long long sg = idx / groups;  // s * N + g
  const int pos = (int)(sg / N);
  const float2* tb = table + (long long)pos * (D / 2) + i0;
  float2 cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = tb[e];
  for (int b = 0; b < B; ++b) {
    const long long off = ((long long)b * S * N + sg) * D + i0;
    const U4 xa = ldg16(src + off), xb = ldg16(src + off + D / 2);
    const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w}, wb[4] = {xb.x, xb.y, xb.z, xb.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float2 r0 = rope_rot(bf16lo(wa[q]), bf16lo(wb[q]), cs[2 * q]);
      const float2 r1 = rope_rot(bf16hi(wa[q]), bf16hi(wb[q]), cs[2 * q + 1]);
      ya[q] = pack_bf16x2(r0.x, r1.x);
      yb[q] = pack_bf16x2(r0.y, r1.y);
    }
    stg16(dst + off, U4{ya[0], ya[1], ya[2], ya[3]});
    stg16(dst + off + D / 2, U4{yb[0], yb[1], yb[2], yb[3]});
  }
}

// The same rotation with the angle table made on the way (one launch instead of two): the threads
// of a work-group cover the (s, g, 8-pair group) items first .. first+255, i.e. positions p0 .. p1;
// they evaluate those positions' (cos, sin) once each (rope_cs, the table kernel's formula, so the
// bits are the same), keep them in LDS for their own rotations and write them to `table` for the
// prefill's q rotation. Entries of a position shared by two work-groups are written by both with
// the same value. LDS: (p1 - p0 + 1) * D/2 <= (255 / (N * D/16) + 2) * D/2 <= 2040 + D entries.
constexpr int kTableRotMaxD = 512;
constexpr int kTableRotLds = 2040 + kTableRotMaxD;
__global__ __launch_bounds__(256) void rope_table_rotate_bf16_kernel(const uint16_t* __restrict__ src,
                                                                     uint16_t* __restrict__ dst,
                                                                     float2* __restrict__ table, int B, int S,
                                                                     int N, int D, double neg2_log2theta_over_d,
                                                                     unsigned int* __restrict__ zero) {
  __shared__ float2 cs_lds[kTableRotLds];
  if (zero != nullptr && blockIdx.x == 0 && threadIdx.x < 128) zero[threadIdx.x] = 0u;
  const int half = D / 2, groups = D / 16;
  const long long total = (long long)S * N * groups;
  const long long first = (long long)blockIdx.x * 256;
  const long long last = min(first + 255, total - 1);
  const int p0 = (int)(first / groups / N), p1 = (int)(last / groups / N);
  const int nent = (p1 - p0 + 1) * half;
  for (int e = threadIdx.x; e < nent; e += 256) {
    const int pos = p0 + e / half, i = e % half;
    const float2 c = rope_cs(pos, i, neg2_log2theta_over_d);
    cs_lds[e] = c;
    table[(long long)pos * half + i] = c;
  }
  __syncthreads();
  const long long idx = first + threadIdx.x;
  if (idx >= total) return;
  const int i0 = (int)(idx % groups) * 8;
  const long long sg = idx / groups;  // s * N + g
  const int pos = (int)(sg / N);
  const float2* tb = cs_lds + (pos - p0) * half + i0;
  float2 cs[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) cs[e] = tb[e];
  for (int b = 0; b < B; ++b) {
    const long long off = ((long long)b * S * N + sg) * D + i0;
    const U4 xa = ldg16(src + off), xb = ldg16(src + off + D / 2);
    const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w}, wb[4] = {xb.x, xb.y, xb.z, xb.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float2 r0 = rope_rot(bf16lo(wa[q]), bf16lo(wb[q]), cs[2 * q]);
      const float2 r1 = rope_rot(bf16hi(wa[q]), bf16hi(wb[q]), cs[2 * q + 1]);
      ya[q] = pack_bf16x2(r0.x, r1.x);
      yb[q] = pack_bf16x2(r0.y, r1.y);
    }
    stg16(dst + off, U4{ya[0], ya[1], ya[2], ya[3]});
    stg16(dst + off + D / 2, U4{yb[0], yb[1], yb[2], yb[3]});
  }
}

// Copy of src [rows, D] into dst with the half-split pairs of the span [roff, roff + Dr) rotated by
// the table [S][Dr/2] (row r has position (r / N) % S); the dims before the span are copied (the
// span ends the row, roff + Dr = D). Used for MLA's decoupled RoPE block ("Transformer 与 LLM" slide 06: only the 64-dim k^R / q^R part carries
// position). 16-byte vectors throughout: per row, roff/8 threads copy 8 dims each and Dr/16 threads
// each rotate 8 pairs (i, i + Dr/2), reading both halves and writing both (rows of 16-byte-aligned
// pitch; D, roff multiples of 8 and Dr of 16, checked by the launcher).
__global__ void rope_span_table_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                       const float2* __restrict__ table, long long rows, int S, int N, int D,
                                       int roff, int Dr) {
  const int ncopy = roff / 8, nrot = Dr / 16, half = Dr / 2;
  const int groups = ncopy + nrot;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * groups) return;
  const long long row = idx / groups;
  const int gi = (int)(idx % groups);
  const uint16_t* x = src + row * D;
  uint16_t* y = dst + row * D;
  if (gi < ncopy) {
    stg16(y + 8 * gi, ldg16(x + 8 * gi));
    return;
  }
  const int i0 = 8 * (gi - ncopy);  // pairs i0 .. i0+7 of the span
  const int pos = (int)((row / N) % S);
  const float2* tb = table + (long long)pos * half + i0;
  const U4 xa = ldg16(x + roff + i0), xb = ldg16(x + roff + half + i0);
  const uint32_t wa[4] = {xa.x, xa.y, xa.z, xa.w}, wb[4] = {xb.x, xb.y, xb.z, xb.w};
  uint32_t ya[4], yb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float2 r0 = rope_rot(bf16lo(wa[q]), bf16lo(wb[q]), tb[2 * q]);
    const float2 r1 = rope_rot(bf16hi(wa[q]), bf16hi(wb[q]), tb[2 * q + 1]);
    ya[q] = pack_bf16x2(r0.x, r1.x);
    yb[q] = pack_bf16x2(r0.y, r1.y);
  }
  stg16(y + roff + i0, U4{ya[0], ya[1], ya[2], ya[3]});
  stg16(y + roff + half + i0, U4{yb[0], yb[1], yb[2], yb[3]});
}

hipError_t launch_rope_span_table(const uint16_t* src, uint16_t* dst, const float2* table, long long rows, int S,
                                  int N, int D, int roff, int Dr, hipStream_t st) {
  // the span is the row's trailing block (MLA: 128 + 64 = 192): nothing after it to copy
  if (D % 8 != 0 || roff % 8 != 0 || Dr % 16 != 0 || roff + Dr != D || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return hipErrorInvalidValue;
  const long long n = rows * (roff / 8 + Dr / 16);
  if (n == 0) return hipSuccess;
  rope_span_table_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(src, dst, table, rows, S, N, D,
                                                                                   roff, Dr);
  return hipGetLastError();
}

// In-place rotation with explicit positions; fp64 angle and fp64 rotation, one rounding at the
// store. One thread per pair.
template <typename T>
__global__ void rope_apply_kernel(T* __restrict__ x, const int* __restrict__ positions, long long rows,
                                  int S, int N, int D, double neg2_log2theta_over_d, int interleaved) {
  const int half = D / 2;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * half) return;
  const long long row = idx / half;
  const int i = (int)(idx % half);
  const long long tok = row / N;  // b * S + s
  const int pos = positions ? positions[tok] : (int)(tok % S);
  const double inv_freq = exp2(neg2_log2theta_over_d * (double)i);
  double s, c;
  sincos((double)pos * inv_freq, &s, &c);
  T* p = x + row * D;
  const int ia = interleaved ? 2 * i : i;
  const int ib = interleaved ? 2 * i + 1 : i + half;
  const double a = (double)to_f32(p[ia]);
  const double b = (double)to_f32(p[ib]);
  p[ia] = from_f32<T>((float)(a * c - b * s));
  p[ib] = from_f32<T>((float)(a * s + b * c));
}

// KV-cache append with RoPE fused ("Transformer 架构完全深度解析" §九: new K/V are concatenated to
// the cache; K is rotated at its absolute position first, "2.7 ..." §4, "Transformer 架构快速入门"
// §8.2 for a rotary span of Dr <= D dims). Token s of sequence b goes to cache row
// t = start[b] + s (clamped to max_ctx - S). One thread per (token, 8 consecutive dims), looping
// over the KV heads: the (cos, sin) of its dims' pairs are computed once per token, not per head.
// It copies those 8 dims of V, and of K outside the rotary span; inside it, each output element
// is its pair's rotation (rope_cs / rope_rot, the same bits as the prefill's key pre-pass).
// kVec: every pointer and row pitch allows 16-byte accesses, so the 8 dims move as one vector.
template <bool kVec>
__global__ void kv_append_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                 uint16_t* __restrict__ kc, uint16_t* __restrict__ vc,
                                 const int* __restrict__ start, int B, int S, int Nkv, int D, int max_ctx,
                                 long long ldk, long long ldv, double neg2_log2theta_over_dr, int rope, int Dr,
                                 int interleaved) {
  const int groups = D / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)B * S * groups) return;
  const int d0 = (int)(idx % groups) * 8;
  const long long tok = idx / groups;  // b * S + s
  const int s = (int)(tok % S);
  const int b = (int)(tok / S);
  const int t = min(max(start[b], 0), max_ctx - S) + s;
  const int half = Dr / 2;
  // per dim: rotated or copied; the pair (da, db) holding it and whether it is the pair's first
  float2 cs[8];
  int partner[8];
  bool rot[8], first[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    rot[e] = rope && d < Dr;
    first[e] = interleaved ? (d & 1) == 0 : d < half;
    const int da = first[e] ? d : (interleaved ? d - 1 : d - half);
    partner[e] = first[e] ? (interleaved ? da + 1 : da + half) : da;
    cs[e] = rot[e] ? rope_cs(t, interleaved ? da / 2 : da, neg2_log2theta_over_dr) : make_float2(1.f, 0.f);
  }
  for (int g = 0; g < Nkv; ++g) {
    const long long row = tok * Nkv + g;
    const uint16_t* kx = k_new + row * D;
    const uint16_t* vx = v_new + row * D;
    uint16_t* ky = kc + ((long long)b * max_ctx + t) * Nkv * ldk + (long long)g * ldk;
    uint16_t* vy = vc + ((long long)b * max_ctx + t) * Nkv * ldv + (long long)g * ldv;
    uint16_t own[8], res[8];
    if constexpr (kVec) {
      stg16(vy + d0, ldg16(vx + d0));
      const U4 w = ldg16(kx + d0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) own[e] = (uint16_t)(ws[e >> 1] >> (16 * (e & 1)));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vy[d0 + e] = vx[d0 + e];
        own[e] = kx[d0 + e];
      }
    }
    // partners of a fully rotated group: inside its own chunk (adjacent pairs), or one 16-byte chunk
    // half a span away (half-split with half % 8 == 0); otherwise one element at a time
    uint16_t pv[8];
    const bool grp = kVec && rope && d0 + 8 <= Dr && (interleaved || half % 8 == 0);
    if (grp) {
      if (interleaved) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = own[e ^ 1];
      } else {
        const U4 w2 = ldg16(kx + (d0 < half ? d0 + half : d0 - half));
        const uint32_t ps[4] = {w2.x, w2.y, w2.z, w2.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = (uint16_t)(ps[e >> 1] >> (16 * (e & 1)));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!rot[e]) {
        res[e] = own[e];
        continue;
      }
      const uint16_t other = grp ? pv[e] : kx[partner[e]];
      const float2 r = first[e] ? rope_rot(bf16_to_f32(own[e]), bf16_to_f32(other), cs[e])
                                : rope_rot(bf16_to_f32(other), bf16_to_f32(own[e]), cs[e]);
      res[e] = f32_to_bf16(first[e] ? r.x : r.y);
    }
    if constexpr (kVec) {
      stg16(ky + d0, U4{res[0] | (uint32_t(res[1]) << 16), res[2] | (uint32_t(res[3]) << 16),
                        res[4] | (uint32_t(res[5]) << 16), res[6] | (uint32_t(res[7]) << 16)});
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) ky[d0 + e] = res[e];
    }
  }
}

hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* kc, uint16_t* vc,
                            const int* start, int B, int S, int Nkv, int D, int max_ctx, long long ldk, long long ldv,
                            double theta, int Dr, int interleaved, hipStream_t st) {
  const long long n = (long long)B * S * (D / 8);
  if (n == 0) return hipSuccess;
  const bool rope = theta > 0.0;
  const double k = rope ? -2.0 * log2(theta) / (double)Dr : 0.0;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool vec = a16(k_new) && a16(v_new) && a16(kc) && a16(vc) && ldk % 8 == 0 && ldv % 8 == 0;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (vec)
    kv_append_kernel<true><<<grid, block, 0, st>>>(k_new, v_new, kc, vc, start, B, S, Nkv, D, max_ctx, ldk, ldv, k,
                                                   rope ? 1 : 0, Dr, interleaved ? 1 : 0);
  else
    kv_append_kernel<false><<<grid, block, 0, st>>>(k_new, v_new, kc, vc, start, B, S, Nkv, D, max_ctx, ldk, ldv, k,
                                                    rope ? 1 : 0, Dr, interleaved ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* table, int S, int D, double theta, hipStream_t st) {
  const long long n = (long long)S * (D / 2);
  if (n == 0) return hipSuccess;
  const double k = -2.0 * log2(theta) / (double)D;
  rope_table_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(table, S, D / 2, k);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_rotate_table(const T* src, T* dst, const float2* table, long long rows, int S, int N,
                                    int D, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (D % 16 == 0 && rows % ((long long)S * N) == 0) {
      const long long n = (long long)S * N * (D / 16);
      if (n == 0) return hipSuccess;
      rope_rotate_table_bf16_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(
          reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst), table, (int)(rows / ((long long)S * N)),
          S, N, D);
      return hipGetLastError();
    }
  }
  const long long n = rows * (D / 16);
  if (n == 0) return hipSuccess;
  rope_rotate_table_kernel<T><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(src, dst, table, rows,
                                                                                       S, N, D);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_apply(T* x, const int* positions, long long rows, int S, int N, int D, double theta,
                             int interleaved, hipStream_t st) {
  const long long n = rows * (D / 2);
  if (n == 0) return hipSuccess;
  const double k = -2.0 * log2(theta) / (double)D;
  rope_apply_kernel<T><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(x, positions, rows, S, N, D, k,
                                                                                interleaved);
  return hipGetLastError();
}

template hipError_t launch_rope_rotate_table<float>(const float*, float*, const float2*, long long, int, int, int,
                                                    hipStream_t);
template hipError_t launch_rope_rotate_table<bf16_t>(const bf16_t*, bf16_t*, const float2*, long long, int, int,
                                                     int, hipStream_t);

hipError_t launch_rope_table_rotate_bf16(const bf16_t* src, bf16_t* dst, float2* table, int B, int S, int N, int D,
                                         double theta, hipStream_t st, unsigned int* zero, bool* zeroed) {
  if (zeroed != nullptr) *zeroed = false;
  if (D % 16 != 0 || D > kTableRotMaxD || D <= 0 || B <= 0 || S <= 0 || N <= 0) {  // the two-launch form
    hipError_t e = launch_rope_table(table, S, D, theta, st);
    if (e != hipSuccess) return e;
    return launch_rope_rotate_table<bf16_t>(src, dst, table, (long long)B * S * N, S, N, D, st);
  }
  const long long n = (long long)S * N * (D / 16);
  const double k = -2.0 * log2(theta) / (double)D;
  rope_table_rotate_bf16_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st>>>(
      reinterpret_cast<const uint16_t*>(src), reinterpret_cast<uint16_t*>(dst), table, B, S, N, D, k, zero);
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess && zeroed != nullptr) *zeroed = zero != nullptr;
  return e;
}
template hipError_t launch_rope_apply<float>(float*, const int*, long long, int, int, int, double, int,
                                             hipStream_t);
template hipError_t launch_rope_apply<bf16_t>(bf16_t*, const int*, long long, int, int, int, double, int,
                                              hipStream_t);

}  // namespace attn
