// KV-cache decode for MHA/GQA/MQA on gfx950, split over the context ("split-KV"), plus the
// reduction that merges the splits.
//
// What is computed: for each sequence b and query head h, the single new query attends to the
// cached keys 0 .. ctx_b-1 of KV head h / (Nh/Nkv) with no mask ("Transformer 架构完全深度解析"
// §九: the new K/V are appended first; "Transformer 架构快速入门" §13.2).
//
// Decode streams the cache once and does ~4 FLOP per byte, so it is bound by HBM bandwidth:
//   - a work-group owns (b, a group of up to 8 query heads sharing one KV head, one context
//     chunk); every cached row is read by exactly one work-group, with 128-bit loads by 16
//     lanes per 256-byte row, several rows in flight per lane;
//   - pass 1 streams K and forms q.k with bf16 dot2 instructions (exact bf16 products) and a
//     16-lane DPP reduction; pass 2 takes the chunk's max and exp2 once per score (no running
//     rescale inside a chunk); pass 3 streams V and accumulates p.v;
//   - each chunk writes (max, sum, unnormalised output) in fp32; the reduction kernel merges
//     the chunks with the online-softmax algebra ("Transformer 架构完全深度解析" §十三: the
//     running max / sum recurrences, applied to whole chunks).
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // quad xor 1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // quad xor 2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
  return x;
}

// Pairwise sums over rows (0,1),(2,3) then lanes (l, l^32): the whole-wave sum of the four rows.
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  return pair_sum32(x);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int DPL>
struct Vec;  // DPL bf16 elements = DPL/2 dwords
template <>
struct Vec<8> {
  uint32_t d[4];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const U4 v = ldg16(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
};
template <>
struct Vec<4> {
  uint32_t d[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    d[0] = v.x; d[1] = v.y;
  }
};

template <int D, int HG>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int DPL = D / 16;  // dims per lane: one row per 16 lanes
  constexpr int NDW = DPL / 2;
  extern __shared__ float smem[];
  float* sc = smem;  // [chunk][HG] scores, then probabilities
  __shared__ float red[4][HG][D];
  __shared__ float mls[HG][2];

  const int tid = threadIdx.x;
  const int n_hg = a.Nh / HG;
  const int s = blockIdx.x % a.nsplit;
  const int hgrp = (blockIdx.x / a.nsplit) % n_hg;
  const int b = blockIdx.x / (a.nsplit * n_hg);
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int t0 = s * a.chunk;
  if (t0 >= ctx) return;  // empty split: the reduction ignores it
  const int t1 = min(ctx, t0 + a.chunk);
  const int n = t1 - t0;
  const int h0 = hgrp * HG;
  const int g = h0 / (a.Nh / a.Nkv);
  const int lg = tid >> 4, li = tid & 15;
  const int w = tid >> 6, lane = tid & 63;

  // ---- query (optionally rotated at position ctx-1), kept as bf16 pairs for dot2 ----
  uint32_t qv[HG][NDW];
#pragma unroll
  for (int hl = 0; hl < HG; ++hl) {
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h0 + hl) * D;
    Vec<DPL> mine;
    mine.load(qp + li * DPL);
    if (a.rope_theta > 0) {
      const bool first = li * DPL < D / 2;
      Vec<DPL> other;
      other.load(qp + (first ? li * DPL + D / 2 : li * DPL - D / 2));
      const double k2 = -2.0 * log2(a.rope_theta) / (double)D;
#pragma unroll
      for (int e = 0; e < NDW; ++e) {
        float r[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int dim = li * DPL + 2 * e + hf;
          const int i = first ? dim : dim - D / 2;
          double sn, cs;
          sincos((double)(ctx - 1) * exp2(k2 * (double)i), &sn, &cs);
          const double x = hf ? bf16hi(mine.d[e]) : bf16lo(mine.d[e]);
          const double y = hf ? bf16hi(other.d[e]) : bf16lo(other.d[e]);
          r[hf] = first ? (float)(x * cs - y * sn) : (float)(y * sn + x * cs);
        }
        qv[hl][e] = pack_bf16x2(r[0], r[1]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < NDW; ++e) qv[hl][e] = mine.d[e];
    }
  }

  const long long row_k = (long long)a.Nkv * a.ldk;
  const long long row_v = (long long)a.Nkv * a.ldv;
  const uint16_t* kb = a.kc + ((long long)b * a.max_ctx * a.Nkv + g) * a.ldk + li * DPL;
  const uint16_t* vb = a.vc + ((long long)b * a.max_ctx * a.Nkv + g) * a.ldv + li * DPL;

  // ---- pass 1: scores x = scale*log2(e) * q.k ----
  for (int base = t0 + lg; base < t1; base += 16 * kUnroll) {
    Vec<DPL> kr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + 16 * u;
      if (t < t1) kr[u].load(kb + t * row_k);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + 16 * u;
      if (t < t1) {
#pragma unroll
        for (int hl = 0; hl < HG; ++hl) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < NDW; ++e)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qv[hl][e]),
                                                  __builtin_bit_cast(bf16x2, kr[u].d[e]), acc, false);
          acc = row16_sum(acc);
          if (li == 0) sc[(t - t0) * HG + hl] = acc * a.scale_log2;
        }
      }
    }
  }
  __syncthreads();

  // ---- pass 2: chunk max and sum per head; scores become probabilities ----
  for (int hl = w; hl < HG; hl += 4) {
    float mx = -INFINITY;
    for (int i = lane; i < n; i += 64) mx = fmaxf(mx, sc[i * HG + hl]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float pr = fast_exp2(sc[i * HG + hl] - mx);
      sc[i * HG + hl] = pr;
      sum += pr;
    }
    sum = wave_sum(sum);
    if (lane == 0) {
      mls[hl][0] = mx;
      mls[hl][1] = sum;
    }
  }
  __syncthreads();

  // ---- pass 3: o = sum_t p_t v_t ----
  float o[HG][DPL];
#pragma unroll
  for (int hl = 0; hl < HG; ++hl)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hl][e] = 0.f;
  for (int base = t0 + lg; base < t1; base += 16 * kUnroll) {
    Vec<DPL> vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + 16 * u;
      if (t < t1) vr[u].load(vb + t * row_v);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + 16 * u;
      if (t < t1) {
        float vf[DPL];
#pragma unroll
        for (int e = 0; e < NDW; ++e) {
          vf[2 * e] = bf16lo(vr[u].d[e]);
          vf[2 * e + 1] = bf16hi(vr[u].d[e]);
        }
#pragma unroll
        for (int hl = 0; hl < HG; ++hl) {
          const float pr = sc[(t - t0) * HG + hl];
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[hl][e] = fmaf(pr, vf[e], o[hl][e]);
        }
      }
    }
  }

  // ---- reduce the 16 row groups of the work-group, write the partial ----
#pragma unroll
  for (int hl = 0; hl < HG; ++hl)
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[hl][e] = rows_sum(o[hl][e]);
  if (lane < 16) {
#pragma unroll
    for (int hl = 0; hl < HG; ++hl)
#pragma unroll
      for (int e = 0; e < DPL; ++e) red[w][hl][li * DPL + e] = o[hl][e];
  }
  __syncthreads();
  for (int i = tid; i < HG * D; i += kThreads) {
    const int hl = i / D, d = i % D;
    const float tot = red[0][hl][d] + red[1][hl][d] + red[2][hl][d] + red[3][hl][d];
    const long long slot = ((long long)b * a.Nh + h0 + hl) * a.nsplit + s;
    a.part_o[slot * D + d] = tot;
    if (d == 0) {
      a.part_ml[slot * 2 + 0] = mls[hl][0];
      a.part_ml[slot * 2 + 1] = mls[hl][1];
    }
  }
}

// Merge the chunks of each (b, h): m* = max m_s, l* = sum 2^(m_s - m*) l_s,
// out = sum 2^(m_s - m*) o_s / l*. One wave per (b, h).
__global__ __launch_bounds__(kThreads) void decode_reduce_kernel(DecodeArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= a.B * a.Nh) return;
  const int b = wid / a.Nh;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int ns = (ctx + a.chunk - 1) / a.chunk;
  const long long slot0 = (long long)wid * a.nsplit;
  const int Dv = a.Dv;
  uint16_t* op = a.out + (long long)wid * Dv;
  if (ns == 0) {
    for (int d = lane; d < Dv; d += 64) op[d] = 0;
    return;
  }
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.part_ml[(slot0 + s) * 2]);
  float l = 0.f;
  for (int s = 0; s < ns; ++s) l += fast_exp2(a.part_ml[(slot0 + s) * 2] - mx) * a.part_ml[(slot0 + s) * 2 + 1];
  const float inv = 1.f / l;
  for (int d = lane; d < Dv; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < ns; ++s) acc += fast_exp2(a.part_ml[(slot0 + s) * 2] - mx) * a.part_o[(slot0 + s) * Dv + d];
    op[d] = f32_to_bf16(acc * inv);
  }
}

template <int D, int HG>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  const long long n_wg = (long long)a.B * (a.Nh / HG) * a.nsplit;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = (size_t)a.chunk * HG * sizeof(float);
  decode_split_kernel<D, HG><<<dim3((unsigned)n_wg), dim3(kThreads), lds, st>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Nh / a.Nkv;
  if (G % 8 == 0) return launch_t<D, 8>(a, st);
  if (G % 4 == 0) return launch_t<D, 4>(a, st);
  if (G % 2 == 0) return launch_t<D, 2>(a, st);
  return launch_t<D, 1>(a, st);
}
}  // namespace

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t st) {
  switch (a.Dqk) {
    case 64:
      return launch_d<64>(a, st);
    case 128:
      return launch_d<128>(a, st);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t st) {
  const long long waves = (long long)a.B * a.Nh;
  if (waves == 0) return hipSuccess;
  decode_reduce_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace attn
