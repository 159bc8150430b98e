// MLA-absorbed decode on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// What is computed ("Transformer 与 LLM：结构、实现与算量" slide 06): after W_UK and W_UV are
// absorbed, decode is multi-query attention in which all query heads share ONE cached row per
// token, [c^KV (512) ; k^R (64)]. Scores use all 576 dims, the value is the latent part c^KV
// (the first 512 dims of the same row), and the scale is given by the caller (1/sqrt(192) for
// DeepSeek-V3's 128 + 64 per-head query dims).
//
// With 128 heads per row the work is ~242 FLOP per cached byte, so the matrix cores are used:
//   - a work-group = NW waves x 16 heads owns (sequence, 16*NW heads, one context chunk); with
//     NW = 8 all 128 heads share the work-group, so every cached row crosses HBM once per chunk;
//   - 32-token tiles (36 KiB) go from HBM straight into an LDS ring of NB stages
//     (global_load_lds_dwordx4): the loads of tiles j+1 .. j+NB-1 are in flight while tile j is
//     computed;
//     16-byte chunks are XOR-swizzled within aligned groups of 8 by bits of the row index so
//     the operand reads below are free of bank conflicts;
//   - per wave and tile: S^T[32 tokens x 16 heads] = K Q^T (18 k-steps over 576 dims, K operand
//     read row-major), online softmax per head, then O^T[512 x 16] += V^T P^T (32 MFMAs) with the
//     V operand read from the SAME row-major tile by the transposing LDS read (4 consecutive
//     tokens of one dim per lane) - the row serves as K and as V without a second copy;
//   - each chunk writes (max, sum, unnormalised output) in fp32 for the split reduction; a single
//     chunk writes the normalised bf16 output directly.
// Work-group ids are mapped so that the head groups of one (sequence, chunk) run on one XCD and
// share its L2 when the heads do not fit one work-group.
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int DQ = 576;
constexpr int DV = 512;
constexpr int TT = 32;            // tokens per tile
constexpr int TILE = TT * DQ;     // elements per tile (36 KiB)
constexpr int NSLOT = TILE * 2 / 1024;  // 36 load instructions of 1 KiB per tile
constexpr int NKK = DQ / 32;      // 18 k-steps
constexpr int NDB = DV / 16;      // 32 output blocks of 16 dims
constexpr int NB = 2;             // LDS ring stages (tiles in flight: NB - 1)

// XOR key applied to the 16-byte chunk index in tile row `row`: bits 1-2 of the row, so a chunk
// stays inside its aligned group of 8 (72 chunks per row). gfx950 serves a 128-bit LDS read in four
// passes of 16 lanes (the lanes with equal bit 5 and equal parity of bits 2-4) and a 64-bit read in
// two passes of 32 lanes; with this key the K operand reads (16 consecutive rows, one chunk per
// 16-lane row group) and the transposing V reads (8 rows x 32 bytes per pass) hit 16 distinct
// 16-byte bank groups per pass, i.e. no bank conflicts. (The 1152-byte row pitch puts odd rows
// half a bank line away from even rows.)
__device__ __forceinline__ int rkey(int row, int /*chunk*/) { return row & 6; }

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
__global__ __launch_bounds__(NW * 64, (NW >= 8 ? 2 : 1)) void decode_mla_kernel(DecodeArgs a) {
  constexpr int NT = NW * 64;
  constexpr int SPW = (NSLOT + NW - 1) / NW;  // load slots per wave (some waves one fewer)
  constexpr int WAITN = NSLOT / NW;           // loads of the next tile every wave has issued
  __shared__ __attribute__((aligned(1024))) uint16_t ring[NB][TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // id -> (pair = (b, split), head group): the head groups of a pair sit 8 ids apart (one XCD)
  const int n_hg = a.Nh / (16 * NW);
  const int n_pairs = a.B * a.nsplit;
  const int id = blockIdx.x;
  const int pair = (id / 8 / n_hg) * 8 + id % 8;
  const int hgrp = (id / 8) % n_hg;
  if (pair >= n_pairs) return;
  const int b = pair / a.nsplit;
  const int s = pair % a.nsplit;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int t0 = s * a.chunk;
  if (t0 >= ctx) return;
  const int t1 = min(ctx, t0 + a.chunk);
  const int hc = lane & 15, rg = lane >> 4;  // head column, row group
  const int h = hgrp * 16 * NW + w * 16 + hc;

  // Q^T operand: head h, dims kk*32 + rg*8 .. +7
  bf16x8 qreg[NKK];
  {
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h) * DQ + rg * 8;
    U4 raw[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) raw[kk] = ldg16(qp + kk * 32);
    if (a.rope_theta > 0) {
      // decoupled RoPE on the q^R block (dims 512..575, slide 06 of "Transformer 与 LLM"): half-split
      // pairs (512 + i, 544 + i), frequency theta^(-2i/64), position ctx-1; the cache holds rotated
      // k^R. Dims 512 + rg*8 + j sit in raw[16], their partners in raw[17] of the same lane.
      const double k2 = -2.0 * log2(a.rope_theta) / (double)(DQ - DV);
      uint32_t* pa = &raw[DV / 32].x;
      uint32_t* pb = &raw[DV / 32 + 1].x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float ra[2], rb[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int i = rg * 8 + 2 * e + hf;
          double sn, cs;
          sincos((double)(ctx - 1) * exp2(k2 * (double)i), &sn, &cs);
          const double x = hf ? bf16hi(pa[e]) : bf16lo(pa[e]);
          const double y = hf ? bf16hi(pb[e]) : bf16lo(pb[e]);
          ra[hf] = (float)(x * cs - y * sn);
          rb[hf] = (float)(x * sn + y * cs);
        }
        pa[e] = pack_bf16x2(ra[0], ra[1]);
        pb[e] = pack_bf16x2(rb[0], rb[1]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
    retire_vmem();
  }

  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4{};
  float m = -INFINITY, lsum = 0.f;

  // ---- per-lane LDS offsets (elements) ----
  // K operand (row hc of a 16-token group, logical chunk 4*kk + rg). The physical chunk is
  // 4*(kk ^ (key>>2)) + ((rg ^ key) & 3): one base per kk mod 4 plus 32*(kk & ~3) elements.
  const int kkey = rkey(hc, 0);
  int koff[4];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) koff[m4] = hc * DQ + ((4 * m4 + rg) ^ kkey) * 8;
  // V operand (transposing read): 16-lane group rg addresses token rows rg*4 + j (and +16), dims
  // db*16 + 4c, logical chunk 2*db + (c>>1): physical 2*(db ^ (key>>1)) + (((c>>1) ^ key) & 1).
  const int tj = (lane & 15) >> 2, tc = lane & 3;
  const int vrow = rg * 4 + tj;
  const int vkey = rkey(vrow, 0);
  const int vbase = vrow * DQ + ((((tc >> 1) ^ vkey) & 1) * 8) + (tc & 1) * 4;
  const int vx = vkey >> 1;

  // ---- tile loads: wave w fills slots w, w+NW, ...; lane i of slot sl covers tile bytes
  // sl*1024 + 16*i = row*1152 + 16*pc and fetches logical chunk pc ^ rkey(row, pc) of that row ----
  const long long row_pitch = a.ldk;  // Nkv == 1
  const uint16_t* seq = a.kc + (long long)b * a.max_ctx * row_pitch;
  auto issue_tile = [&](int j, uint16_t* dst) {
#pragma unroll
    for (int r = 0; r < SPW; ++r) {
      const int sl = w + NW * r;
      if (sl < NSLOT) {
        const int ob = sl * 1024 + 16 * lane;
        const int row = ob / (DQ * 2);
        const int pc = (ob % (DQ * 2)) / 16;
        const int t = min(t0 + j * TT + row, t1 - 1);  // rows past the chunk re-read a valid row (masked)
        load_lds16_async(seq + t * row_pitch + (pc ^ rkey(row, pc)) * 8, dst + sl * 512);
      }
    }
  };

  auto compute_tile = [&](int j, const uint16_t* Tt) {
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const int ko = koff[kk & 3] + 32 * (kk & ~3);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Tt + tg * 16 * DQ + ko);
        sacc[tg] = mfma16x16x32(ka, qreg[kk], sacc[tg]);
      }
      if (kk % 3 == 2) __builtin_amdgcn_sched_barrier(0);  // bound how far LDS reads are hoisted
    }
    const int tbase = t0 + j * TT;
    if (tbase + TT > t1) {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tbase + tg * 16 + rg * 4 + i >= t1) sacc[tg][i] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3]));
    mt = fmaxf(mt, fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mt = rows_max(mt);
    // lazy reference max (moves only when a head's max grows by more than 2^8; see prefill)
    const float mb = mt * a.scale_log2;
    const bool move = mb > m + 8.f;
    const float m_new = move ? mb : m;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = move ? fast_exp2(m - m_use) : 1.f;
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
    lsum = fmaf(lsum, alpha, psum);
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[db][i] *= alpha;
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, U4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int vo = vbase + 16 * ((db & ~7) + ((db & 7) ^ vx));
      const uint2 lo = lds_read_tr16(Tt + vo);
      const uint2 hi = lds_read_tr16(Tt + 16 * DQ + vo);
      const bf16x8 va = __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[db], 0, 0, 0);
      if (db % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int n_tiles = (t1 - t0 + TT - 1) / TT;
  auto wait_tile = [&](int j) {  // this wave's loads of tile j done; those of later tiles may fly
    const int later = min(n_tiles - 1 - j, NB - 2);
    if (later >= 2)
      wait_vmem_n<(2 * WAITN <= 63 ? 2 * WAITN : WAITN)>();  // the smaller count over-waits safely
    else if (later == 1)
      wait_vmem_n<WAITN>();
    else
      wait_vmem();
    barrier_only();
  };

#pragma unroll
  for (int j = 0; j < NB - 1; ++j)
    if (j < n_tiles) issue_tile(j, ring[j]);
  for (int j = 0; j < n_tiles; ++j) {
    wait_tile(j);
    if (j + NB - 1 < n_tiles) issue_tile(j + NB - 1, ring[(j + NB - 1) % NB]);
    compute_tile(j, ring[j % NB]);
  }

  // ---- result: lane holds head hc, dims db*16 + rg*4 .. +3 ----
  const float ltot = rows_sum(lsum);
  if (a.nsplit == 1) {
    const float inv = 1.f / ltot;
    uint16_t* op = a.out + ((long long)b * a.Nh + h) * DV + rg * 4;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<uint2*>(op + db * 16) =
          make_uint2(pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv));
    return;
  }
  const long long slot = ((long long)b * a.Nh + h) * a.nsplit + s;
  float* po = a.part_o + slot * DV + rg * 4;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<float4*>(po + db * 16) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
  if (rg == 0) {
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = ltot;
  }
}

template <int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t st) {
  const long long n_hg = a.Nh / (16 * NW);
  const long long pairs = (long long)a.B * a.nsplit;
  const long long n_wg = ((pairs + 7) / 8) * 8 * n_hg;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  decode_mla_kernel<NW><<<dim3((unsigned)n_wg), dim3(NW * 64), 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace

int mla_waves_per_group(int Nh) { return Nh % 128 == 0 ? 8 : Nh % 64 == 0 ? 4 : Nh % 32 == 0 ? 2 : 1; }

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
  switch (mla_waves_per_group(a.Nh)) {
    case 8:
      return launch_nw<8>(a, st);
    case 4:
      return launch_nw<4>(a, st);
    case 2:
      return launch_nw<2>(a, st);
    default:
      return launch_nw<1>(a, st);
  }
}

}  // namespace attn
