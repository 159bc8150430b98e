// bf16 causal prefill on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// What is computed: out = softmax(scale * Q K^T + M) V per (batch, query head), "Transformer 架构
// 快速入门" §4, with query head h reading KV head h / (Nh/Nkv) (same page, §6.3).
//
// Work decomposition (one 256-thread work-group = 4 waves):
//   - a work-group owns BP consecutive query positions of HPW query heads that share one KV head
//     (HPW = 4 for GQA groups of 4: the K/V tile staged in LDS is used by all four heads, so K/V
//     are never replicated per head - the logical sharing of "Transformer 架构快速入门" §6.3);
//   - each wave owns 32 query rows of one head and computes the transposed score block
//     S^T = K Q^T, so that one lane holds one query's scores: the row max needs a single
//     lane-pair exchange and the row sum none until the end;
//   - K/V tiles of 64 keys are loaded with 128-bit coalesced loads into registers one tile
//     ahead, then stored to a double-buffered LDS tile (V transposed on the way, so that the
//     P.V contraction reads 4 consecutive keys per 8-byte LDS read);
//   - tiles past the work-group's last query are never visited and 32-key blocks above a wave's
//     diagonal are skipped ("2.7 Transformer Decoder Block完整解析" §3.3); the element mask is
//     applied only on blocks that cross the diagonal or the sequence end;
//   - online softmax over tiles ("Transformer 架构完全深度解析" §十三: running max and sum; the
//     output accumulator is rescaled by the same factor, and only when some row's max moved).
// Grid order puts the work-groups with the most tiles first.
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kBC = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t sel_lo(uint32_t x, uint32_t y) { return __byte_perm(x, y, 0x5410); }
__device__ __forceinline__ uint32_t sel_hi(uint32_t x, uint32_t y) { return __byte_perm(x, y, 0x7632); }
__device__ __forceinline__ uint32_t dw(const U4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, const float2* __restrict__ table, int B, int S, int Nh, int Nkv, float c,
    int causal, int n_ptiles) {
  constexpr int BP = 32 * (4 / HPW);        // query positions per work-group
  constexpr int KP = D + 8;                 // K tile row pitch (elements)
  constexpr int VP = kBC + 4;               // transposed V row pitch (elements)
  constexpr int OCT = D / 8;                // 16-byte chunks per row
  constexpr int NKC = kBC * OCT / kThreads; // K chunks per thread
  constexpr int NVU = (kBC / 4) * OCT;      // V units of 4 keys x 8 dims
  constexpr int NQ = D / 16;                // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;               // 32-row blocks of the output's head dim

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBC * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VP];

  const int tid = threadIdx.x;
  const int HGn = Nh / HPW;
  const int id = blockIdx.x;
  const int bh = id % (B * HGn);
  const int pt = n_ptiles - 1 - id / (B * HGn);
  const int b = bh / HGn;
  const int h0 = (bh % HGn) * HPW;
  const int g = h0 / (Nh / Nkv);
  const int p0 = pt * BP;
  const int w = tid >> 6, lane = tid & 63;
  const int h = h0 + (w % HPW);
  const int wp0 = p0 + (w / HPW) * 32;
  const int col = lane & 31, hh = lane >> 5;
  const int p = wp0 + col;  // this lane's query position

  // ---- Q^T operand in registers (RoPE applied here when a table is given) ----
  bf16x8 qreg[NQ];
  {
    U4 raw[NQ];
    if (p < S) {
      const uint16_t* qp = q + (((long long)b * S + p) * Nh + h) * D + hh * 8;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = ldg16(qp + kk * 16);
      if (table) {
        const float2* tb = table + (long long)p * (D / 2) + hh * 8;
#pragma unroll
        for (int kk = 0; kk < NQ / 2; ++kk) {
          U4& ra = raw[kk];
          U4& rb = raw[kk + NQ / 2];
          uint32_t na[4], nb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 c0 = tb[kk * 16 + 2 * e], c1 = tb[kk * 16 + 2 * e + 1];
            const float a0 = bf16lo(dw(ra, e)), a1 = bf16hi(dw(ra, e));
            const float b0 = bf16lo(dw(rb, e)), b1 = bf16hi(dw(rb, e));
            na[e] = pack_bf16x2(a0 * c0.x - b0 * c0.y, a1 * c1.x - b1 * c1.y);
            nb[e] = pack_bf16x2(a0 * c0.y + b0 * c0.x, a1 * c1.y + b1 * c1.x);
          }
          ra = U4{na[0], na[1], na[2], na[3]};
          rb = U4{nb[0], nb[1], nb[2], nb[3]};
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = U4{0, 0, 0, 0};
    }
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m = -INFINITY;  // running max of scale*log2(e)*score for this lane's query
  float lsum = 0.f;     // running sum over the keys this lane holds

  const long long kv_stride = (long long)Nkv * D;
  const uint16_t* kbase = k + ((long long)b * S * Nkv + g) * D;
  const uint16_t* vbase = v + ((long long)b * S * Nkv + g) * D;

  U4 kreg[NKC];
  U4 vreg[4];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < NKC; ++r) {
      const int ch = tid + kThreads * r;
      const int key = j * kBC + ch / OCT;
      kreg[r] = key < S ? ldg16(kbase + key * kv_stride + (ch % OCT) * 8) : U4{0, 0, 0, 0};
    }
    if (tid < NVU) {
      const int kq = tid / OCT, oc = tid % OCT;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j * kBC + kq * 4 + r;
        vreg[r] = key < S ? ldg16(vbase + key * kv_stride + oc * 8) : U4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NKC; ++r) {
      const int ch = tid + kThreads * r;
      *reinterpret_cast<U4*>(&Ks[buf][(ch / OCT) * KP + (ch % OCT) * 8]) = kreg[r];
    }
    if (tid < NVU) {
      const int kq = tid / OCT, oc = tid % OCT;
      const int unit = kq ^ (oc & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x0 = dw(vreg[0], e), x1 = dw(vreg[1], e), x2 = dw(vreg[2], e), x3 = dw(vreg[3], e);
        uint2 lo = make_uint2(sel_lo(x0, x1), sel_lo(x2, x3));
        uint2 hi = make_uint2(sel_hi(x0, x1), sel_hi(x2, x3));
        *reinterpret_cast<uint2*>(&Vt[buf][(oc * 8 + 2 * e) * VP + unit * 4]) = lo;
        *reinterpret_cast<uint2*>(&Vt[buf][(oc * 8 + 2 * e + 1) * VP + unit * 4]) = hi;
      }
    }
  };

  const int last = causal ? min(S, p0 + BP) : S;
  const int n_tiles = (last + kBC - 1) / kBC;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    // ---- S^T = K Q^T for the two 32-key blocks of this tile ----
    f32x16 sacc[2];
    bool active[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = j * kBC + kb * 32;
      active[kb] = kb0 < S && (!causal || kb0 <= wp0 + 31);
      sacc[kb] = f32x16{};
      if (active[kb]) {
        const uint16_t* kr = &Ks[buf][(kb * 32 + col) * KP + hh * 8];
#pragma unroll
        for (int kk = 0; kk < NQ; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kr + kk * 16);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[kb], 0, 0, 0);
        }
      }
    }

    // ---- mask, running max, probabilities ----
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kb0 = j * kBC + kb * 32;
      if (active[kb]) {
        const bool need_mask = (causal && kb0 + 31 > wp0) || (kb0 + 32 > S);
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb0 + (i >> 2) * 8 + hh * 4 + (i & 3);
            if (key >= S || (causal && key > p)) sacc[kb][i] = -INFINITY;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = -INFINITY;
      }
    }
    mt = pair_max32(mt);
    const float m_new = fmaxf(m, mt * c);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;

    uint32_t pk[2][2][4];  // [key block][k-step][dword] bf16 probabilities
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(fmaf(sacc[kb][i], c, -m_use));
        const float e1 = fast_exp2(fmaf(sacc[kb][i + 1], c, -m_use));
        psum += e0 + e1;
        pk[kb][i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
      }
    }
    lsum = lsum * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!active[kb]) continue;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 bop = __builtin_bit_cast(bf16x8, U4{pk[kb][s][0], pk[kb][s][1], pk[kb][s][2], pk[kb][s][3]});
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int dim = db * 32 + col;
          const int sw = (dim >> 3) & 15;
          const uint16_t* row = &Vt[buf][dim * VP];
          const uint2 lo = *reinterpret_cast<const uint2*>(row + ((kb * 8 + 4 * s + hh) ^ sw) * 4);
          const uint2 hi = *reinterpret_cast<const uint2*>(row + ((kb * 8 + 4 * s + 2 + hh) ^ sw) * 4);
          const bf16x8 aop = __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, o[db], 0, 0, 0);
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, round to bf16, store BSHD ----
  const float inv = 1.f / pair_sum32(lsum);
  if (p < S) {
    uint16_t* op = out + (((long long)b * S + p) * Nh + h) * D + hh * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const uint2 wv = make_uint2(pack_bf16x2(o[db][g4 * 4 + 0] * inv, o[db][g4 * 4 + 1] * inv),
                                    pack_bf16x2(o[db][g4 * 4 + 2] * inv, o[db][g4 * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + db * 32 + g4 * 8) = wv;
      }
  }
}

template <int D, int HPW>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int BP = 32 * (4 / HPW);
  const int n_ptiles = (a.S + BP - 1) / BP;
  const long long n_wg = (long long)n_ptiles * a.B * (a.Nh / HPW);
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  prefill_bf16_kernel<D, HPW><<<dim3((unsigned)n_wg), dim3(kThreads), 0, st>>>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
      static_cast<uint16_t*>(a.out), a.table, a.B, a.S, a.Nh, a.Nkv, a.scale_log2, a.causal, n_ptiles);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Nh / a.Nkv;
  if (G % 4 == 0) return launch_t<D, 4>(a, st);
  if (G % 2 == 0) return launch_t<D, 2>(a, st);
  return launch_t<D, 1>(a, st);
}
}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
  switch (a.D) {
    case 64:
      return launch_d<64>(a, st);
    case 128:
      return launch_d<128>(a, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace attn
