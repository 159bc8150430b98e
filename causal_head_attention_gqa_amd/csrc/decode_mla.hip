// MLA-absorbed decode on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed ("Transformer 与 LLM：结构、实现与算量" slide 06): after W_UK and W_UV are
// absorbed, decode is multi-query attention in which all query heads share ONE cached row per
// token, [c^KV (512) ; k^R (64)]. Scores use all 576 dims, the value is the latent part c^KV
// (the first 512 dims of the same row), and the scale is given by the caller (1/sqrt(192) for
// DeepSeek-V3's 128 + 64 per-head query dims).
//
// With 128 heads per row the work is ~242 FLOP per cached byte, so the matrix cores are used:
//   - a work-group = 4 waves x 16 heads owns (b, 64 heads, one context chunk); each cached row
//     is loaded once per work-group with 128-bit coalesced loads (4 rows per thread unit, one
//     tile of 32 tokens ahead in registers) into a double-buffered LDS tile: row-major for the
//     scores and transposed (dims x tokens) for the value contraction;
//   - per wave and tile: S^T[32 tokens x 16 heads] = K Q^T (18 k-steps over 576 dims), online
//     softmax per head, then O^T[512 x 16] += V^T P^T (32 MFMAs);
//   - each chunk writes (max, sum, unnormalised output) in fp32 for the shared split reduction.
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int DQ = 576;
constexpr int DV = 512;
constexpr int TT = 32;          // tokens per tile
constexpr int KP = DQ + 8;      // row-major tile pitch (elements)
constexpr int VP = TT + 4;      // transposed tile pitch (elements)
constexpr int OCT = DQ / 8;     // 72 16-byte chunks per row
constexpr int NUNIT = (TT / 4) * OCT;  // 576 load units of 4 tokens x 8 dims
constexpr int NKK = DQ / 32;    // 18 k-steps
constexpr int NDB = DV / 16;    // 32 output blocks of 16 dims

__device__ __forceinline__ uint32_t sel_lo(uint32_t x, uint32_t y) { return __byte_perm(x, y, 0x5410); }
__device__ __forceinline__ uint32_t sel_hi(uint32_t x, uint32_t y) { return __byte_perm(x, y, 0x7632); }
__device__ __forceinline__ uint32_t dw(const U4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Max / sum over the four 16-lane rows that hold one head's tokens.
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max32(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
}

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void decode_mla_kernel(DecodeArgs a) {
  constexpr int NT = NW * 64;
  constexpr int UPT = (NUNIT + NT - 1) / NT;  // load units per thread
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][TT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][DV * VP];

  const int tid = threadIdx.x;
  const int n_hg = a.Nh / (16 * NW);
  const int s = blockIdx.x % a.nsplit;
  const int hgrp = (blockIdx.x / a.nsplit) % n_hg;
  const int b = blockIdx.x / (a.nsplit * n_hg);
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int t0 = s * a.chunk;
  if (t0 >= ctx) return;
  const int t1 = min(ctx, t0 + a.chunk);
  const int w = tid >> 6, lane = tid & 63;
  const int hc = lane & 15, rg = lane >> 4;  // head column, row group
  const int h = hgrp * 16 * NW + w * 16 + hc;

  // Q^T operand: head h, dims kk*32 + rg*8 .. +7
  bf16x8 qreg[NKK];
  {
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h) * DQ + rg * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = as_bf16x8(ldg16(qp + kk * 32));
  }

  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4{};
  float m = -INFINITY, lsum = 0.f;

  const long long row = a.ldk;  // Nkv == 1
  const uint16_t* base = a.kc + (long long)b * a.max_ctx * row;

  U4 lr[UPT][4];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < UPT; ++r) {
      const int u = tid + NT * r;
      if (u < NUNIT) {
        const int tq = u / OCT, oc = u % OCT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = t0 + j * TT + tq * 4 + e;
          lr[r][e] = t < t1 ? ldg16(base + t * row + oc * 8) : U4{0, 0, 0, 0};
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < UPT; ++r) {
      const int u = tid + NT * r;
      if (u < NUNIT) {
        const int tq = u / OCT, oc = u % OCT;
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<U4*>(&Ks[buf][(tq * 4 + e) * KP + oc * 8]) = lr[r][e];
        if (oc < DV / 8) {
          const int unit = tq ^ (oc & 7);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x0 = dw(lr[r][0], e), x1 = dw(lr[r][1], e), x2 = dw(lr[r][2], e), x3 = dw(lr[r][3], e);
            *reinterpret_cast<uint2*>(&Vt[buf][(oc * 8 + 2 * e) * VP + unit * 4]) =
                make_uint2(sel_lo(x0, x1), sel_lo(x2, x3));
            *reinterpret_cast<uint2*>(&Vt[buf][(oc * 8 + 2 * e + 1) * VP + unit * 4]) =
                make_uint2(sel_hi(x0, x1), sel_hi(x2, x3));
          }
        }
      }
    }
  };

  const int n_tiles = (t1 - t0 + TT - 1) / TT;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    // S^T for two 16-token groups: lane holds head hc, tokens tg*16 + rg*4 + i
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[buf][(tg * 16 + hc) * KP + kk * 32 + rg * 8]);
        sacc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[kk], sacc[tg], 0, 0, 0);
      }
    }
    const int tbase = t0 + j * TT;
    float mt = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tbase + tg * 16 + rg * 4 + i >= t1) sacc[tg][i] = -INFINITY;
        mt = fmaxf(mt, sacc[tg][i]);
      }
    mt = rows_max(mt);
    const float m_new = fmaxf(m, mt * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    uint32_t pk[4];
    float psum = 0.f;
#pragma unroll
    for (int tg = 0; tg < 2; ++tg)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float e0 = fast_exp2(fmaf(sacc[tg][i], a.scale_log2, -m_use));
        const float e1 = fast_exp2(fmaf(sacc[tg][i + 1], a.scale_log2, -m_use));
        psum += e0 + e1;
        pk[tg * 2 + i / 2] = pack_bf16x2(e0, e1);
      }
    lsum = lsum * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= alpha;
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, U4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dim = db * 16 + hc;
      const int sw = (dim >> 3) & 7;
      const uint16_t* vr = &Vt[buf][dim * VP];
      const uint2 lo = *reinterpret_cast<const uint2*>(vr + ((rg) ^ sw) * 4);
      const uint2 hi = *reinterpret_cast<const uint2*>(vr + ((4 + rg) ^ sw) * 4);
      const bf16x8 va = __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // partial: unnormalised O (lane: head hc, dims db*16 + rg*4 .. +3), max and sum
  const long long slot = ((long long)b * a.Nh + h) * a.nsplit + s;
  float* po = a.part_o + slot * DV + rg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<float4*>(po + db * 16) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
  const float ltot = rows_sum(lsum);
  if (rg == 0) {
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = ltot;
  }
}
}  // namespace

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
  int nw = (a.Nh % 64 == 0) ? 4 : (a.Nh % 32 == 0) ? 2 : 1;
  const long long n_wg = (long long)a.B * (a.Nh / (16 * nw)) * a.nsplit;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  switch (nw) {
    case 4:
      decode_mla_kernel<4><<<dim3((unsigned)n_wg), dim3(256), 0, st>>>(a);
      break;
    case 2:
      decode_mla_kernel<2><<<dim3((unsigned)n_wg), dim3(128), 0, st>>>(a);
      break;
    default:
      decode_mla_kernel<1><<<dim3((unsigned)n_wg), dim3(64), 0, st>>>(a);
      break;
  }
  return hipGetLastError();
}

}  // namespace attn
