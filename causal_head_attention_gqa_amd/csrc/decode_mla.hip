// MLA-absorbed decode on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16).
//
// What is computed ("Transformer 与 LLM：结构、实现与算量" slide 06): after W_UK and W_UV are
// absorbed, decode is multi-query attention in which all query heads share ONE cached row per
// token, [c^KV (512) ; k^R (64)]. Scores use all 576 dims, the value is the latent part c^KV
// (the first 512 dims of the same row), and the scale is given by the caller (1/sqrt(192) for
// DeepSeek-V3's 128 + 64 per-head query dims).
//
// With 128 heads per row the work is ~242 FLOP per cached byte, so the matrix cores are used. Three
// kernels: head counts that are multiples of 128 without in-kernel RoPE use the wide kernel at the
// end of the file (all heads of a row in one work-group, 64 per pair of waves); other multiples of
// 64 use the pair kernel further below (32 heads per pair of waves on 32x32x16 products); other
// head counts use this one, 16 heads per wave:
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
//   - each chunk writes (max, sum) in fp32 and its output normalised by that sum in bf16 for the
//     split reduction; a single
//     chunk writes the normalised bf16 output directly.
// Work-group ids are mapped so that the head groups of one (sequence, chunk) run on one XCD and
// share its L2 when the heads do not fit one work-group.
#include "kernels.hpp"

#include <type_traits>

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

// Angle of the decoupled RoPE at position pos for frequency index f = lane % 32: (sin, cos) of
// pos * theta^(-2f/64) in fp64. One position serves every query head of a sequence, so the 32
// angles are evaluated once per wave (one per lane) and rope_qr_hilo fetches the ones it needs
// from the lanes that hold them; every lane of the wave calls both.
__device__ __forceinline__ void rope_lane_angle(int pos, double theta, double& sn, double& cs) {
  const double k2 = -2.0 * log2(theta) / (double)(DQ - DV);
  sincos((double)pos * exp2(k2 * (double)(threadIdx.x & 31)), &sn, &cs);
}

// decoupled RoPE of one lane's q^R pairs: dims 512 + i held in `a` (i = i0 .. i0+7), their
// half-split partners 544 + i in `b`, rotated by the angles of rope_lane_angle. The rotated fp32
// value x is kept as two bf16 numbers, hi = bf16(x) in a / b and lo = bf16(x - hi) in alo / blo
// (x - hi is exact in fp32): the products then see q^R to ~2^-17 instead of bf16's 2^-9, which
// matters when k^R is large and the softmax is nearly one-hot.
__device__ __forceinline__ void rope_qr_hilo(U4& a, U4& b, U4& alo, U4& blo, int i0, double sn_l, double cs_l) {
  uint32_t* pa = &a.x;
  uint32_t* pb = &b.x;
  uint32_t* la = &alo.x;
  uint32_t* lb = &blo.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float ra[2], rb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const double sn = __shfl(sn_l, i0 + 2 * e + hf), cs = __shfl(cs_l, i0 + 2 * e + hf);
      const double x = hf ? bf16hi(pa[e]) : bf16lo(pa[e]);
      const double y = hf ? bf16hi(pb[e]) : bf16lo(pb[e]);
      ra[hf] = (float)(x * cs - y * sn);
      rb[hf] = (float)(x * sn + y * cs);
    }
    pa[e] = pack_bf16x2(ra[0], ra[1]);
    pb[e] = pack_bf16x2(rb[0], rb[1]);
    la[e] = pack_bf16x2(ra[0] - bf16lo(pa[e]), ra[1] - bf16hi(pa[e]));
    lb[e] = pack_bf16x2(rb[0] - bf16lo(pb[e]), rb[1] - bf16hi(pb[e]));
  }
}

// kRope: rotate q^R in-kernel (a.rope_theta > 0) and add the products of its bf16 residuals.
template <int NW, bool kRope>
__global__ __launch_bounds__(NW * 64, (NW >= 8 ? 2 : 1)) void decode_mla_kernel(DecodeArgs a) {
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
  const int hc = lane & 15, rg = lane >> 4;  // head column, row group
  const int h = hgrp * 16 * NW + w * 16 + hc;
  if (t0 >= ctx) {
    // an empty split; with a single chunk (no merge follows) an empty context gives a zero row
    if (a.nsplit == 1) {
      uint16_t* op = a.out + ((long long)b * a.Nh + h) * DV + rg * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<uint2*>(op + db * 16) = make_uint2(0u, 0u);
    }
    return;
  }
  const int t1 = min(ctx, t0 + a.chunk);

  // Q^T operand: head h, dims kk*32 + rg*8 .. +7
  bf16x8 qreg[NKK];
  bf16x8 qlo[2];  // kRope: bf16 residuals of the rotated q^R (k-steps 16, 17)
  {
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h) * DQ + rg * 8;
    U4 raw[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) raw[kk] = ldg16(qp + kk * 32);
    U4 lo[2] = {U4{0, 0, 0, 0}, U4{0, 0, 0, 0}};
    if (kRope) {
      // decoupled RoPE on the q^R block (dims 512..575, slide 06 of "Transformer 与 LLM"): half-split
      // pairs (512 + i, 544 + i), frequency theta^(-2i/64), position ctx-1; the cache holds rotated
      // k^R. Dims 512 + rg*8 + j sit in raw[16], their partners in raw[17] of the same lane.
      double sn, cs;
      rope_lane_angle(ctx - 1, a.rope_theta, sn, cs);
      rope_qr_hilo(raw[DV / 32], raw[DV / 32 + 1], lo[0], lo[1], rg * 8, sn, cs);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
    qlo[0] = as_bf16x8(lo[0]);
    qlo[1] = as_bf16x8(lo[1]);
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
    if constexpr (kRope) {  // the q^R residuals against k-steps 16 and 17
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kk = NKK - 2 + u;
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Tt + tg * 16 * DQ + koff[kk & 3] + 32 * (kk & ~3));
          sacc[tg] = mfma16x16x32(ka, qlo[u], sacc[tg]);
        }
      }
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
  const long long slot = part_slot(a, b, h, s);
  uint16_t* po = a.part_o + slot * DV + rg * 4;
  const float inv = 1.f / ltot;  // the chunk's output, normalised by its own sum, in bf16
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<uint2*>(po + db * 16) =
        make_uint2(pack_bf16x2(o[db][0] * inv, o[db][1] * inv), pack_bf16x2(o[db][2] * inv, o[db][3] * inv));
  if (rg == 0) {
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = ltot;
  }
}

// ---- 32 heads per wave pair (head counts that are multiples of 64) ----
//
// A work-group = 4 waves (one per SIMD) owns (sequence, 64 heads, one context chunk). Waves 2p and
// 2p+1 form a pair that shares heads 32p .. 32p+31 of the group:
//   - Q.K: wave 2p+r (r = 0, 1) contracts dims 288r .. 288r+287 of its 32 heads against a 32-token
//     tile (S^T = K Q^T on v_mfma_f32_32x32x16_bf16, 18 k-steps), writes the 32x32 partial scores
//     to LDS, and after a barrier adds its partner's: both waves then hold the same full scores
//     (fp32 addition is commutative, so the two sums are bit-identical) and run the same online
//     softmax;
//   - P.V: wave 2p+r accumulates O^T for output dims 256r .. 256r+255 of the pair's 32 heads
//     (16 products per tile, V^T read from the same row-major tile by the transposing LDS read).
// Per lane this needs 72 query registers and 128 accumulator registers, so one wave per SIMD
// keeps everything in registers. Each tile operand read from LDS feeds a 32-wide product, half the
// LDS traffic per FLOP of the 16-heads-per-wave form above, which is bound by those reads.
// The two head groups of a 128-head sequence chunk are dispatched 8 ids apart, i.e. to the same
// XCD at about the same time, so the second read of each cache row is served by that XCD's L2.
namespace pair {
constexpr int kWaves = 4;
constexpr int kHeads = 64;               // heads per work-group
constexpr int kStages = 4;               // LDS ring: tiles j+1 .. j+3 load while j is computed
constexpr int kSPW = NSLOT / kWaves;     // 9 tile-load instructions per wave and tile
constexpr int kHalfQ = DQ / 2;           // 288 reduction dims per wave
constexpr int kKS = kHalfQ / 16;         // 18 k-steps of 16 dims
constexpr int kDB = DV / 2 / 32;         // 8 output blocks of 32 dims per wave
static_assert(NSLOT % kWaves == 0, "tile loads split evenly over the waves");

// XOR key of the 16-byte chunk index in tile row `row` (only the low 3 bits of the chunk change,
// so a chunk stays in its aligned group of 8): row bits 1, 2, 3 -> key bits 2, 1, 0. The 1152-byte
// row pitch puts odd rows half a bank line (128 B) away from even rows. K operand reads (128-bit,
// 32 consecutive rows, one chunk per half-wave): a 16-lane pass covers 16 distinct values of
// row & 15, which the key and the row parity send to 16 distinct 16-byte bank groups.
// Transposing V reads (64-bit, 4 consecutive rows x 64 contiguous bytes per 16-lane group):
// row bit 1 selects the other half of the chunk group and row bit 0 the other half bank line, so
// each 32-lane pass hits 32 distinct 8-byte bank groups.
__device__ __forceinline__ int key(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}

// kRope: rotate q^R in-kernel (a.rope_theta > 0) and add the products of its bf16 residuals.
template <bool kRope>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_mla_pair_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[kStages][TILE];
  __shared__ __attribute__((aligned(16))) float xch[kWaves][4][64][4];  // partial scores per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = w & 1;         // reduction half of Q.K / output half of P.V
  const int hf = lane >> 5;    // half-wave: k-slot group of the MFMA operands
  const int col = lane & 31;   // head within the pair (MFMA column)
  // id -> (pair = (b, split), head group): the head groups of a pair sit 8 ids apart (one XCD)
  const int n_hg = a.Nh / kHeads;
  const int n_pairs = a.B * a.nsplit;
  const int id = blockIdx.x;
  const int sp_id = (id / 8 / n_hg) * 8 + id % 8;
  const int hgrp = (id / 8) % n_hg;
  if (sp_id >= n_pairs) return;
  const int b = sp_id / a.nsplit;
  const int s = sp_id % a.nsplit;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int t0 = s * a.chunk;
  const int h = hgrp * kHeads + (w >> 1) * 32 + col;
  if (t0 >= ctx) {
    // an empty split; with a single chunk (no merge follows) an empty context gives a zero row
    if (a.nsplit == 1) {
      uint16_t* op = a.out + ((long long)b * a.Nh + h) * DV + r * (DV / 2) + hf * 4;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *reinterpret_cast<uint2*>(op + db * 32 + g * 8) = make_uint2(0u, 0u);
    }
    return;
  }
  const int t1 = min(ctx, t0 + a.chunk);

  // Q^T operand of k-step kk: head h, dims 288r + 16kk + 8hf .. +7
  bf16x8 qreg[kKS];
  bf16x8 qlo[4];  // kRope, upper half: bf16 residuals of the rotated q^R (k-steps 14..17)
  {
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h) * DQ + r * kHalfQ + hf * 8;
    U4 raw[kKS];
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) raw[kk] = ldg16(qp + kk * 16);
    U4 lo[4] = {U4{0, 0, 0, 0}, U4{0, 0, 0, 0}, U4{0, 0, 0, 0}, U4{0, 0, 0, 0}};
    if (kRope && r == 1) {
      // q^R = dims 512..575 = k-steps 14..17 of the upper half: dims 512 + 16u + 8hf + j in
      // raw[14 + u], their partners 544 + 16u + 8hf + j in raw[16 + u]
      double sn, cs;
      rope_lane_angle(ctx - 1, a.rope_theta, sn, cs);
      rope_qr_hilo(raw[14], raw[16], lo[0], lo[2], hf * 8, sn, cs);
      rope_qr_hilo(raw[15], raw[17], lo[1], lo[3], 16 + hf * 8, sn, cs);
    }
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
#pragma unroll
    for (int u = 0; u < 4; ++u) qlo[u] = as_bf16x8(lo[u]);
    retire_vmem();  // from here on only the tile loads count in vmcnt
  }

  f32x16 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) o[i] = f32x16{};
  float m = 0.f, lsum = 0.f;
  bool ovf = false;
  constexpr float kOvf = 1.8446744e19f;  // 2^64

  // ---- per-lane LDS offsets (elements) ----
  // K operand of k-step kk: row col, logical chunk c0 + 2kk with c0 = 36r + hf; the key changes
  // only the low 3 bits, so (c0 + 2(kk&3) + 8(kk>>2)) ^ key = ((c0 + 2(kk&3)) ^ key) + 8(kk>>2).
  const int kkey = key(col);
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = col * DQ + (((36 * r + hf + 2 * u) ^ kkey) << 3);
  // V operand (transposing read) of (ks, t, db): 16-lane group (dq, hf), lane (tj, tc) addresses
  // row 16ks + 8t + 4hf + tj, dims 256r + 32db + 16dq + 4tc, i.e. logical chunk
  // 32r + 4db + x with x = 2dq + (tc >> 1). The row's key is (tj>>1)<<2 | hf<<1 | t, so the physical
  // chunk is 32r + 4(db ^ (tj>>1)) + (x ^ 2hf ^ t): one register per (db parity, t) plus an
  // immediate (16ks + 8t) * 576 + 32 (db & ~1).
  const int tj = (lane & 15) >> 2, tc = lane & 3, dq = (lane >> 4) & 1;
  const int x = 2 * dq + (tc >> 1);
  int vb[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      vb[par][t] = (4 * hf + tj) * DQ + 8 * (32 * r + 4 * (par ^ (tj >> 1)) + (x ^ (2 * hf) ^ t)) + (tc & 1) * 4;

  // ---- tile loads: wave w fills slots w*9 .. w*9+8; lane i of slot sl covers tile bytes
  // sl*1024 + 16i = row*1152 + 16pc and fetches logical chunk pc ^ key(row) of that row ----
  const long long ldk = a.ldk;  // Nkv == 1
  const uint16_t* seq = a.kc + (long long)b * a.max_ctx * ldk;
  int lrow[kSPW], lchk[kSPW];
#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    const int ob = (w * kSPW + u) * 1024 + 16 * lane;
    lrow[u] = ob / (DQ * 2);
    lchk[u] = ((ob % (DQ * 2)) / 16) ^ key(ob / (DQ * 2));
  }
  const int n_tiles = (t1 - t0 + TT - 1) / TT;
  auto issue_tile = [&](int j, uint16_t* dst) {
    const int tb = t0 + j * TT;
#pragma unroll
    for (int u = 0; u < kSPW; ++u) {
      const int t = min(tb + lrow[u], t1 - 1);  // rows past the chunk re-read a valid row (masked)
      load_lds16_async<false>(seq + (long long)t * ldk + lchk[u] * 8, dst + (w * kSPW + u) * 512);
    }
  };

  auto compute_tile = [&](int j, const uint16_t* T) {
    // partial S^T[32 tokens x 32 heads] over this wave's 288 dims: one accumulation chain (a wave
    // issues dependent 32x32x16 products at the full rate, and a second chain would cost 32 AGPR
    // reads and 16 adds per tile to combine) and kKR K operands in flight
    constexpr int kKR = 4;
    auto kread = [&](int kk) { return *reinterpret_cast<const bf16x8*>(T + koff[kk & 3] + 64 * (kk >> 2)); };
    bf16x8 ka[kKR];
#pragma unroll
    for (int u = 0; u < kKR; ++u) ka[u] = kread(u);
    f32x16 sv = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKR], qreg[kk], sv, 0, 0, 0);
      if (kk + kKR < kKS) ka[kk % kKR] = kread(kk + kKR);
    }
    if constexpr (kRope) {
      // the q^R residuals against the same K operands, still in the ring (k-steps 14..17)
      if (r == 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[(kKS - 4 + u) % kKR], qlo[u], sv, 0, 0, 0);
      }
    }
    // exchange with the partner wave (w ^ 1): same lane = same head and tokens
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4*>(&xch[w][g][lane][0]) = f32x4{sv[4 * g], sv[4 * g + 1], sv[4 * g + 2], sv[4 * g + 3]};
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 pv = *reinterpret_cast<const f32x4*>(&xch[w ^ 1][g][lane][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * g + i] += pv[i];
    }
    // token of score i: tile base + 8(i>>2) + 4hf + (i&3)
    const int tbase = t0 + j * TT;
    if (tbase + TT > t1) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tbase + (i >> 2) * 8 + hf * 4 + (i & 3) >= t1) sv[i] = -INFINITY;
    }
    // fixed reference max: the first tile's max per head, the only tile whose max is computed; a
    // later score may exceed it by up to ~2^60 (p, the sums and O stay finite in fp32 and bf16). A
    // tile whose exponentials sum past 2^64 in either half of a head flags the head, which is then
    // recomputed exactly after the loop
    if (j == 0) {
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sv[i]);
      m = pair_max32(mt) * a.scale_log2;
    }
    uint32_t pk[2][4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float e0 = fast_exp2(fmaf(sv[i], a.scale_log2, -m));
      const float e1 = fast_exp2(fmaf(sv[i + 1], a.scale_log2, -m));
      psum += e0 + e1;
      pk[i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
    }
    lsum += psum;
    ovf |= !(psum <= kOvf);
    // O^T[256 dims x 32 heads] += V^T P^T; two V operands in flight
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, U4{pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]});
      auto vread = [&](int db) {
        const uint16_t* p = T + (16 * ks) * DQ + 32 * (db & ~1);
        const uint2 lo = lds_read_tr16(p + vb[db & 1][0]);
        const uint2 hi = lds_read_tr16(p + 8 * DQ + vb[db & 1][1]);
        return __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      };
      constexpr int kVR = 4;  // V operands in flight
      bf16x8 va[kVR];
#pragma unroll
      for (int u = 0; u < kVR; ++u) va[u] = vread(u);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db % kVR], bop, o[db], 0, 0, 0);
        if (db + kVR < kDB) va[db % kVR] = vread(db + kVR);
      }
    }
  };

  // ---- ring of 4 stages (three tiles in flight while one is computed, which the cold-cache
  // latency needs); a load past the last tile re-reads the last one into a stage that is
  // never read again, so every step keeps one fixed vmcnt. One loop body with the stage picked by
  // a scalar index: the accumulators then keep one register assignment through the loop. ----
  issue_tile(0, ring[0]);
  issue_tile(min(1, n_tiles - 1), ring[1]);
  issue_tile(min(2, n_tiles - 1), ring[2]);
  int cur = 0;
  for (int j = 0; j < n_tiles; ++j) {
    wait_vmem_n<2 * kSPW>();  // tile j has landed (tiles j+1 and j+2 may still fly)
    barrier_only();
    issue_tile(min(j + 3, n_tiles - 1), ring[(cur + 3) & 3]);
    compute_tile(j, ring[cur]);
    cur = (cur + 1) & 3;
  }
  wait_vmem();  // the re-reads must land before the work-group's LDS is released

  // ---- result: lane holds head h, dims 256r + 32db + 8g + 4hf + i in o[db][4g + i] ----
  const float ltot = pair_sum32(lsum);
  const long long slot = part_slot(a, b, h, s);
  const uint64_t bal = __ballot(ovf);
  uint64_t bad = (bal | (bal >> 32)) & 0xffffffffull;  // heads flagged by either of their lanes
  if (!((bad >> col) & 1)) {
    if (a.nsplit == 1) {
      const float inv = 1.f / ltot;
      uint16_t* op = a.out + ((long long)b * a.Nh + h) * DV + r * (DV / 2) + hf * 4;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(op + db * 32 + g * 8) =
              make_uint2(pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
    } else {
      uint16_t* po = a.part_o + slot * DV + r * (DV / 2) + hf * 4;
      const float inv = 1.f / ltot;  // the chunk's output, normalised by its own sum, in bf16
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<uint2*>(po + db * 32 + g * 8) =
              make_uint2(pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                         pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
      if (r == 0 && hf == 0) {
        a.part_ml[slot * 2 + 0] = m;
        a.part_ml[slot * 2 + 1] = ltot;
      }
    }
  }

  // ---- heads whose scores outgrew the reference max by ~2^60 or more (never for scores of
  // ordinary size): their accumulators may have overflowed, so they are recomputed exactly by a
  // plain two-pass loop over the chunk's rows (vector ALU, blocks of 4096 tokens merged with the
  // same running max / sum algebra). Both waves of a pair see the same scores and flags. ----
  __syncthreads();  // every wave is done with the ring: its LDS holds the recompute's scratch
  if (bad == 0) return;
  float* qs = reinterpret_cast<float*>(&ring[0][0]) + w * (kStages * TILE / 2 / kWaves);  // 576 + 4096 floats
  float* sc = qs + DQ;
  const double k2 = a.rope_theta > 0 ? -2.0 * log2(a.rope_theta) / (double)(DQ - DV) : 0.0;
  for (; bad; bad &= bad - 1) {
    const int c = __builtin_ctzll(bad);
    const int hc = hgrp * kHeads + (w >> 1) * 32 + c;
    const uint16_t* qp = a.q + ((long long)b * a.Nh + hc) * DQ;
    for (int d = lane; d < DQ; d += 64) {
      float v = bf16_to_f32(qp[d]);
      if (a.rope_theta > 0 && d >= DV) {  // the decoupled RoPE of the main path, kept in fp32 here
        const int i = (d - DV) & 31;
        double sn, cs;
        sincos((double)(ctx - 1) * exp2(k2 * (double)i), &sn, &cs);
        const double x = bf16_to_f32(qp[DV + i]), y = bf16_to_f32(qp[DV + 32 + i]);
        v = (float)(d < DV + 32 ? x * cs - y * sn : x * sn + y * cs);
      }
      qs[d] = v;
    }
    float mr = -INFINITY, lr = 0.f, o4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int tb = t0; tb < t1; tb += 4096) {
      const int n = min(4096, t1 - tb);
      float mx = -INFINITY;
      for (int i = lane; i < n; i += 64) {
        const uint16_t* kp = seq + (long long)(tb + i) * ldk;
        float acc = 0.f;
        for (int d = 0; d < DQ; d += 8) {
          const U4 kv = ldg16(kp + d);
          acc = fmaf(qs[d + 0], bf16lo(kv.x), acc);
          acc = fmaf(qs[d + 1], bf16hi(kv.x), acc);
          acc = fmaf(qs[d + 2], bf16lo(kv.y), acc);
          acc = fmaf(qs[d + 3], bf16hi(kv.y), acc);
          acc = fmaf(qs[d + 4], bf16lo(kv.z), acc);
          acc = fmaf(qs[d + 5], bf16hi(kv.z), acc);
          acc = fmaf(qs[d + 6], bf16lo(kv.w), acc);
          acc = fmaf(qs[d + 7], bf16hi(kv.w), acc);
        }
        acc *= a.scale_log2;
        sc[i] = acc;
        mx = fmaxf(mx, acc);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(mr, mx);
      const float al = mr == -INFINITY ? 0.f : fast_exp2(mr - mn);
      lr *= al;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] *= al;
      mr = mn;
      for (int i = 0; i < n; ++i) {
        const float pw = fast_exp2(sc[i] - mr);
        lr += pw;
        const uint2 vv = *reinterpret_cast<const uint2*>(seq + (long long)(tb + i) * ldk + r * (DV / 2) + 4 * lane);
        o4[0] = fmaf(pw, bf16lo(vv.x), o4[0]);
        o4[1] = fmaf(pw, bf16hi(vv.x), o4[1]);
        o4[2] = fmaf(pw, bf16lo(vv.y), o4[2]);
        o4[3] = fmaf(pw, bf16hi(vv.y), o4[3]);
      }
    }
    if (a.nsplit == 1) {
      const float inv = 1.f / lr;
      *reinterpret_cast<uint2*>(a.out + ((long long)b * a.Nh + hc) * DV + r * (DV / 2) + 4 * lane) =
          make_uint2(pack_bf16x2(o4[0] * inv, o4[1] * inv), pack_bf16x2(o4[2] * inv, o4[3] * inv));
    } else {
      const long long sl = part_slot(a, b, hc, s);
      const float inv = 1.f / lr;
      *reinterpret_cast<uint2*>(a.part_o + sl * DV + r * (DV / 2) + 4 * lane) =
          make_uint2(pack_bf16x2(o4[0] * inv, o4[1] * inv), pack_bf16x2(o4[2] * inv, o4[3] * inv));
      if (r == 0 && lane == 0) {
        a.part_ml[sl * 2 + 0] = mr;
        a.part_ml[sl * 2 + 1] = lr;
      }
    }
  }
}

hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const long long n_hg = a.Nh / kHeads;
  const long long pairs = (long long)a.B * a.nsplit;
  const long long n_wg = ((pairs + 7) / 8) * 8 * n_hg;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.rope_theta > 0)
    decode_mla_pair_kernel<true><<<dim3((unsigned)n_wg), dim3(kWaves * 64), 0, st>>>(a);
  else
    decode_mla_pair_kernel<false><<<dim3((unsigned)n_wg), dim3(kWaves * 64), 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace pair

// ---- 64 heads per wave pair, all 128 heads of a row in one work-group (head counts that are
// multiples of 128) ----
//
// The pair kernel above reads every V operand from LDS for one 32-head product and exchanges fp32
// partial scores. Here the accumulators of a wave cover 64 heads, so each V operand feeds two
// products:
//   - a work-group = 4 waves owns (sequence, 128 heads, one context chunk); waves 2p and 2p+1 share
//     heads 64p .. 64p+63. Wave 2p+r contracts all 576 dims of its own 32 heads 64p+32r .. +31
//     (36 products per tile, 144 query registers per lane), makes their P in bf16, and swaps it with
//     its partner through LDS; it then accumulates O^T for output dims 256r .. 256r+255 of all 64
//     heads (32 products per tile; 256 accumulator registers, the whole accumulator file);
//   - this fits one wave per SIMD only because nothing but the matrix products touches the
//     accumulators inside the loop: the reference max per head is fixed at the first tile, so no
//     rescale is ever applied to O (heads whose scores outgrow it are recomputed exactly after the
//     loop, as in the pair kernel);
//   - per tile and work-group the LDS carries 144 KiB of K reads, 64 KiB of transposing V reads,
//     8 KiB of P written and read, and the 36 KiB tile itself, for 128 heads; the pair kernel needs
//     as many K reads, twice the V reads and 32 KiB of partial scores for the same heads, and each
//     cached row crosses HBM once here instead of twice;
//   - a 4-stage LDS ring (144 KiB) plus two 8 KiB P buffers;
//   - the chunks of one sequence are dispatched to one XCD (ids of equal id % 8), so the query rows
//     every chunk re-reads stay in that XCD's L2.
namespace wide {
constexpr int kWaves = 4;
constexpr int kHeads = 128;           // heads per work-group
constexpr int kStages = 4;            // tile j (V) and j+1 (K) are read while j+2 and j+3 load
constexpr int kSPW = NSLOT / kWaves;  // 9 tile-load instructions per wave and tile
constexpr int kKS = DQ / 16;          // 36 k-steps of Q.K
constexpr int kDB = DV / 2 / 32;      // 8 output blocks of 32 dims per wave
static_assert(NSLOT % kWaves == 0, "tile loads split evenly over the waves");

// kRope: rotate q^R in-kernel (a.rope_theta > 0) and add the products of its bf16 residuals.
template <bool kRope>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_mla_wide_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint16_t ring[kStages][TILE];
  __shared__ __attribute__((aligned(16))) uint32_t xp[2][kWaves][2][64][4];  // P (bf16 pairs), two buffers

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = w & 1;      // output half of P.V; the pair's head group this wave owns
  const int hf = lane >> 5;
  const int col = lane & 31;
  // id -> (sequence, chunk, head group); ids of equal id % 8 share an XCD and hold all the chunks
  // (and head groups) of sequences id % 8, id % 8 + 8, ...
  const int n_hg = a.Nh / kHeads;
  const int id = blockIdx.x;
  const int kx = id / 8;
  const int hgrp = kx % n_hg;
  const int k2 = kx / n_hg;
  const int b = id % 8 + 8 * (k2 / a.nsplit);
  const int s = k2 % a.nsplit;
  if (b >= a.B) return;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  const int t0 = s * a.chunk;
  const int hp = hgrp * kHeads + (w >> 1) * 64;  // the pair's heads: hp + 32g + col, g = 0, 1
  if (t0 >= ctx) {
    if (a.nsplit == 1) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint16_t* op = a.out + ((long long)b * a.Nh + hp + 32 * g + col) * DV + r * (DV / 2) + hf * 4;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) *reinterpret_cast<uint2*>(op + db * 32 + e * 8) = make_uint2(0u, 0u);
      }
    }
    return;
  }
  const int t1 = min(ctx, t0 + a.chunk);

  // ---- tile loads: wave w fills slots w*9 .. w*9+8; lane i of slot sl covers tile bytes
  // sl*1024 + 16i = row*1152 + 16pc and fetches logical chunk pc ^ key(row) of that row. One
  // byte offset per slot serves the full tiles; the chunk's last, partial tile clamps its rows.
  // The cache rows are read once: non-temporal loads (the query rows, read by every chunk of the
  // sequence, keep the default policy). ----
  const long long ldk = a.ldk;  // Nkv == 1
  const uint16_t* seq = a.kc + (long long)b * a.max_ctx * ldk;
  auto slot_row = [&](int u) { return ((w * kSPW + u) * 1024 + 16 * lane) / (DQ * 2); };
  auto slot_chunk = [&](int u) {
    const int ob = (w * kSPW + u) * 1024 + 16 * lane;
    return ((ob % (DQ * 2)) / 16) ^ pair::key(ob / (DQ * 2));
  };
  uint32_t loff[kSPW];
#pragma unroll
  for (int u = 0; u < kSPW; ++u) loff[u] = 2u * (uint32_t)(slot_row(u) * (int)ldk + slot_chunk(u) * 8);
  const int n_tiles = (t1 - t0 + TT - 1) / TT;
  auto issue_tile = [&](int j, uint16_t* dst) {
    const int tb = t0 + j * TT;
    const uint16_t* base = seq + (long long)tb * ldk;  // wave-uniform (scalar registers)
    const int lim = t1 - 1 - tb;                       // last row of the tile inside the chunk
    // each path starts with 5 wait states, so no branch into it can bring a base that a vector
    // instruction wrote just before the first load (the pair is written by scalar instructions)
    if (lim >= TT - 1) {
      asm volatile("s_nop 4" ::: "memory");
#pragma unroll
      for (int u = 0; u < kSPW; ++u) load_lds16_async_sv<true>(base, loff[u], dst + (w * kSPW + u) * 512);
    } else {
      asm volatile("s_nop 4" ::: "memory");
#pragma unroll
      for (int u = 0; u < kSPW; ++u) {
        const int row = slot_row(u);  // rows past the chunk re-read row lim (masked)
        const uint32_t off = row <= lim ? loff[u] : loff[u] - 2u * (uint32_t)((row - lim) * (int)ldk);
        load_lds16_async_sv<true>(base, off, dst + (w * kSPW + u) * 512);
      }
    }
  };
  // Q^T operand of k-step kk: own head hp + 32r + col, dims 16kk + 8hf .. +7. The wave's 32 query
  // rows are 36 KiB of contiguous memory: they go through the ring first, in the byte layout of a
  // tile (swizzled 16-byte chunks, whole rows per load instruction instead of 32-byte pieces of 32
  // rows), and are read out with the K operand pattern. Load slot u lands in stage u & 3 at 1-KiB
  // column 9w + (u >> 2): exactly the columns this wave's own tile loads fill later, so no other
  // wave writes them and the tile loads may start as soon as this wave has read its rows.
  bf16x8 qreg[kKS];
  {
    const uint16_t* qrows = a.q + ((long long)b * a.Nh + hp + 32 * r) * DQ;  // wave-uniform
    asm volatile("s_nop 4" ::: "memory");
#pragma unroll
    for (int u = 0; u < NSLOT; ++u) {
      const int ob = u * 1024 + 16 * lane;
      const int row = ob / (DQ * 2);
      const uint32_t off = 2u * (uint32_t)(row * DQ + ((((ob % (DQ * 2)) / 16) ^ pair::key(row)) << 3));
      load_lds16_async_sv(qrows, off, &ring[u & 3][0] + (kSPW * w + (u >> 2)) * 512);
    }
    retire_vmem();  // this wave's query rows have landed in its columns of the ring
    const int qkey = pair::key(col);
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      const int bq = col * (DQ * 2) + 16 * (8 * (kk >> 2) + ((2 * (kk & 3) + hf) ^ qkey));
      const int u = bq >> 10;
      qreg[kk] = *reinterpret_cast<const bf16x8*>(&ring[u & 3][0] + (kSPW * w + (u >> 2)) * 512 + ((bq & 1023) >> 1));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read out before the tile loads refill the columns
  }
  bf16x8 qlo[4];  // kRope: bf16 residuals of the rotated q^R (k-steps 32..35)
  if constexpr (kRope) {
    // q^R = dims 512..575 = k-steps 32..35: dims 512 + 16u + 8hf + j in qreg[32 + u], their
    // half-split partners 544 + 16u + 8hf + j in qreg[34 + u]
    U4 ra[4], lo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ra[u] = __builtin_bit_cast(U4, qreg[kKS - 4 + u]);
      lo[u] = U4{0, 0, 0, 0};
    }
    double sn, cs;
    rope_lane_angle(ctx - 1, a.rope_theta, sn, cs);
    rope_qr_hilo(ra[0], ra[2], lo[0], lo[2], hf * 8, sn, cs);
    rope_qr_hilo(ra[1], ra[3], lo[1], lo[3], 16 + hf * 8, sn, cs);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qreg[kKS - 4 + u] = as_bf16x8(ra[u]);
      qlo[u] = as_bf16x8(lo[u]);
    }
  }
  issue_tile(0, ring[0]);

  f32x16 o[2][kDB];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < kDB; ++i) o[g][i] = f32x16{};
  float m = 0.f, lsum = 0.f;  // own head: fixed reference max (log2 units) and this lane's sum
  bool ovf = false;
  constexpr float kOvf = 1.8446744e19f;  // 2^64

  // K operand of k-step kk: row col, logical chunk 2kk + hf = 8(kk>>2) + (2(kk&3) + hf); the key
  // changes only the low 3 bits, so the physical chunk is 8(kk>>2) + ((2(kk&3) + hf) ^ key)
  const int kkey = pair::key(col);
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) koff[u] = col * DQ + (((2 * u + hf) ^ kkey) << 3);
  // V operand (transposing read) of (ks, db): as in the pair kernel, output half r
  const int tj = (lane & 15) >> 2, tc = lane & 3, dq = (lane >> 4) & 1;
  const int x = 2 * dq + (tc >> 1);
  int vb[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      vb[par][t] = (4 * hf + tj) * DQ + 8 * (32 * r + 4 * (par ^ (tj >> 1)) + (x ^ (2 * hf) ^ t)) + (tc & 1) * 4;

  // S^T[32 tokens x 32 own heads] of the tile in T over all 576 dims: one accumulation chain,
  // kKR K operands in flight. With kSpread, this wave's 9 loads of a full tile (base, dst) are
  // issued among the products, one after every fourth, so that their issue overlaps the products.
  auto qk = [&](const uint16_t* T, auto spread, const uint16_t* base, uint16_t* dst) {
    constexpr bool kSpread = decltype(spread)::value;
    constexpr int kKR = 4;
    auto kread = [&](int kk) { return *reinterpret_cast<const bf16x8*>(T + koff[kk & 3] + 64 * (kk >> 2)); };
    bf16x8 ka[kKR];
#pragma unroll
    for (int u = 0; u < kKR; ++u) ka[u] = kread(u);
    f32x16 sv = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % kKR], qreg[kk], sv, 0, 0, 0);
      if (kk + kKR < kKS) ka[kk % kKR] = kread(kk + kKR);
      // keeps the read of k-step kk + kKR here: left alone, the scheduler moves each read down to
      // its product and every product then waits for a full LDS round trip
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kSpread) {
        static_assert(kKS == 4 * kSPW, "one load per four products");
        if (kk % 4 == 0) load_lds16_async_sv_nop<true>(base, loff[kk / 4], dst + (w * kSPW + kk / 4) * 512);
      }
    }
    if constexpr (kRope) {
      // the q^R residuals against the K operands of k-steps 32..35, still in the ring
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[(kKS - 4 + u) % kKR], qlo[u], sv, 0, 0, 0);
    }
    return sv;
  };
  using NoSpread = std::integral_constant<bool, false>;
  using Spread = std::integral_constant<bool, true>;
  // scores of tile j past the chunk's end -> -inf (token of score i: 8(i>>2) + 4hf + (i&3))
  auto mask = [&](f32x16& sv, int j) {
    const int tbase = t0 + j * TT;
    if (tbase + TT > t1) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (tbase + (i >> 2) * 8 + hf * 4 + (i & 3) >= t1) sv[i] = -INFINITY;
    }
  };
  // exponentials of the pair (2i, 2i+1) against the reference max, packed to bf16
  auto expo = [&](const f32x16& sv, int i, float& psum) {
    const float e0 = fast_exp2(fmaf(sv[2 * i], a.scale_log2, -m));
    const float e1 = fast_exp2(fmaf(sv[2 * i + 1], a.scale_log2, -m));
    psum += e0 + e1;
    return pack_bf16x2(e0, e1);
  };
  auto put_p = [&](const uint32_t (&pk)[2][4], int buf) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      *reinterpret_cast<uint4*>(&xp[buf][w][ks][lane][0]) = make_uint4(pk[ks][0], pk[ks][1], pk[ks][2], pk[ks][3]);
  };

  // ---- tile 0: scores, the reference max, P ----
  uint32_t pk[2][4];
  // tile 0 has landed; tiles 1 and 2 load during its products (issued only now: when every
  // work-group starts at once, tile 0 then does not share HBM with them)
  wait_vmem_n<0>();
  if (n_tiles > 1) issue_tile(1, ring[1]);
  if (n_tiles > 2) issue_tile(2, ring[2]);
  barrier_only();  // every wave's part of tile 0 is in LDS
  {
    f32x16 sv = qk(ring[0], NoSpread{}, nullptr, nullptr);
    mask(sv, 0);
    float mt = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sv[i]);
    m = pair_max32(mt) * a.scale_log2;  // fixed reference max: the first tile's max per head
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) pk[i >> 2][i & 3] = expo(sv, i, psum);
    lsum += psum;
    ovf |= !(psum <= kOvf);
    put_p(pk, 0);
  }

  // ---- step j: P.V of tile j (P exchanged at the barrier) while the scores and P of tile j+1 are
  // made: Q.K of tile j+1 first, then its exponentials interleaved with the P.V products. One
  // barrier per step: tile j+1 has landed in every wave, every wave's P(j) is in LDS (both waves of
  // a pair read both groups' P(j) from there after Q.K), and every wave is done with stage
  // (j-1) % 4, which the load of tile j+3 then refills. P goes through two LDS buffers: P(j+1) is
  // written while P(j) may still be read by the partner. ----
  for (int j = 0; j < n_tiles; ++j) {
    // tile j+1 has landed (tile j+2, if there is one, may still fly)
    if (j + 2 < n_tiles)
      wait_vmem_n<kSPW>();
    else
      wait_vmem_n<0>();
    barrier_only();
    const bool more = j + 1 < n_tiles;
    // the load of tile j+3: spread over the products of Q.K(j+1) when that tile is full, else
    // issued at once (a partial last tile clamps its rows)
    const int jl = j + 3;
    const bool spread = jl < n_tiles && t0 + jl * TT + TT <= t1;
    if (jl < n_tiles && !spread) issue_tile(jl, ring[jl & 3]);
    f32x16 sn = f32x16{};
    if (spread) {
      sn = qk(ring[(j + 1) & 3], Spread{}, seq + (long long)(t0 + jl * TT) * ldk, ring[(j + 3) & 3]);
      mask(sn, j + 1);
    } else if (more) {
      sn = qk(ring[(j + 1) & 3], NoSpread{}, nullptr, nullptr);
      mask(sn, j + 1);
    }
    // O^T[256 dims x 32 heads] += V^T P^T for both head groups of the pair: each V operand feeds two
    // products (group r = own P, group 1 - r = the partner's); the exponentials of tile j+1 are
    // spread over the first eight product pairs
    const uint16_t* T = ring[j & 3];
    uint32_t pn[2][4];
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // P(j) of both head groups of the pair (waves 2p and 2p+1), read back from LDS only here so
      // that no P registers stay live across Q.K
      const bf16x8 bop0 = *reinterpret_cast<const bf16x8*>(&xp[j & 1][w & ~1][ks][lane][0]);
      const bf16x8 bop1 = *reinterpret_cast<const bf16x8*>(&xp[j & 1][w | 1][ks][lane][0]);
      auto vread = [&](int db) {
        const uint16_t* p = T + (16 * ks) * DQ + 32 * (db & ~1);
        const uint2 lo = lds_read_tr16(p + vb[db & 1][0]);
        const uint2 hi = lds_read_tr16(p + 8 * DQ + vb[db & 1][1]);
        return __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      };
      constexpr int kVR = 2;  // V operands in flight
      bf16x8 va[kVR];
#pragma unroll
      for (int u = 0; u < kVR; ++u) va[u] = vread(u);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db % kVR], bop0, o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db % kVR], bop1, o[1][db], 0, 0, 0);
        if (db + kVR < kDB) va[db % kVR] = vread(db + kVR);
        if (ks == 0) pn[db >> 2][db & 3] = expo(sn, db, psum);
        __builtin_amdgcn_sched_barrier(0);  // V reads kVR products ahead, exponentials among the products
      }
    }
    if (more) {
      lsum += psum;
      ovf |= !(psum <= kOvf);
    }
    put_p(pn, (j + 1) & 1);  // also past the last tile (never read), so the exponentials stay among the products
  }
  wait_vmem();  // (the last step waited for every load already)

  // ---- (max, sum) and the overflow flags of the own heads to the partner, through the last
  // 1,040 bytes of the ring once every wave is done with it ----
  float* xml = reinterpret_cast<float*>(&ring[kStages - 1][0]) + TILE / 2 - 260;  // [wave][max, sum][32]
  uint32_t* xbad = reinterpret_cast<uint32_t*>(xml + kWaves * 2 * 32);            // [wave]
  const float ltot = pair_sum32(lsum);
  const uint64_t bal = __ballot(ovf);
  __syncthreads();
  if (hf == 0) {
    xml[(w * 2 + 0) * 32 + col] = m;
    xml[(w * 2 + 1) * 32 + col] = ltot;
  }
  if (lane == 0) xbad[w] = (uint32_t)((bal | (bal >> 32)) & 0xffffffffull);
  __syncthreads();
  const uint32_t bad_g[2] = {xbad[(w & ~1) + 0], xbad[(w & ~1) + 1]};

  // ---- result: lane holds head hp + 32g + col, dims 256r + 32db + 8e + 4hf + i in o[g][db][4e + i].
  // Staged through this wave's 32 KiB of the (now idle) ring as 64 rows of 256 dims in bf16, so
  // that the stores are whole 512-byte half rows (two heads per store instruction) instead of
  // 8-byte pieces of 32 rows. 16-byte chunk c of row hl sits at chunk c ^ (hl & 31), with its two
  // 8-byte halves swapped when bit 4 of hl is set: the 64-bit writes (32 lanes = 32 rows) and the
  // 128-bit reads (16 lanes = 16 chunks of one row) then hit distinct LDS bank groups. ----
  uint16_t* stg = &ring[0][0] + w * (64 * 256);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int hl = 32 * g + col;
    const float inv = 1.f / xml[(((w & ~1) + g) * 2 + 1) * 32 + col];  // a chunk's output over its own sum
    const int half = hf ^ ((hl >> 4) & 1);
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint2*>(stg + hl * 256 + (((4 * db + e) ^ (hl & 31)) << 3) + (half << 2)) =
            make_uint2(pack_bf16x2(o[g][db][4 * e] * inv, o[g][db][4 * e + 1] * inv),
                       pack_bf16x2(o[g][db][4 * e + 2] * inv, o[g][db][4 * e + 3] * inv));
  }
#pragma unroll 4
  for (int i = 0; i < 32; ++i) {
    const int hl = 2 * i + hf;  // lanes 0-31: row 2i, lanes 32-63: row 2i+1; chunk col of the row
    uint4 v = *reinterpret_cast<const uint4*>(stg + hl * 256 + ((col ^ (hl & 31)) << 3));
    if ((hl >> 4) & 1) v = make_uint4(v.z, v.w, v.x, v.y);
    if ((bad_g[hl >> 5] >> (hl & 31)) & 1) continue;  // recomputed below
    const long long row = (long long)b * a.Nh + hp + hl;
    uint16_t* op = (a.nsplit == 1 ? a.out + row * DV : a.part_o + part_slot(a, b, hp + hl, s) * DV) + r * (DV / 2) + col * 8;
    stg16_nt(op, U4{v.x, v.y, v.z, v.w});  // every work-group writes at once at its end: streaming stores
  }
  if (a.nsplit > 1 && hf == 0 && !((bad_g[r] >> col) & 1)) {
    const long long slot = part_slot(a, b, hp + 32 * r + col, s);
    a.part_ml[slot * 2 + 0] = m;
    a.part_ml[slot * 2 + 1] = xml[(w * 2 + 1) * 32 + col];
  }

  // ---- heads whose scores outgrew the reference max by ~2^60 or more: recomputed exactly by a
  // plain two-pass loop over the chunk's rows (vector ALU, blocks of 4096 tokens), each wave for
  // its 256 output dims of both groups of the pair. ----
  uint64_t bad = (uint64_t)bad_g[0] | ((uint64_t)bad_g[1] << 32);
  __syncthreads();  // every wave is done with the ring: its LDS holds the recompute's scratch
  if (bad == 0) return;
  float* qs = reinterpret_cast<float*>(&ring[0][0]) + w * (kStages * TILE / 2 / kWaves);  // 576 + 4096 floats
  float* sc = qs + DQ;
  const double kf = kRope ? -2.0 * log2(a.rope_theta) / (double)(DQ - DV) : 0.0;
  for (; bad; bad &= bad - 1) {
    const int c = __builtin_ctzll(bad);
    const int hc = hp + c;
    const uint16_t* qp = a.q + ((long long)b * a.Nh + hc) * DQ;
    for (int d = lane; d < DQ; d += 64) {
      float v = bf16_to_f32(qp[d]);
      if (kRope && d >= DV) {  // the decoupled RoPE of the main path, kept in fp32 here
        const int i = (d - DV) & 31;
        double sn, cs;
        sincos((double)(ctx - 1) * exp2(kf * (double)i), &sn, &cs);
        const double x = bf16_to_f32(qp[DV + i]), y = bf16_to_f32(qp[DV + 32 + i]);
        v = (float)(d < DV + 32 ? x * cs - y * sn : x * sn + y * cs);
      }
      qs[d] = v;
    }
    float mr = -INFINITY, lr = 0.f, o4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int tb = t0; tb < t1; tb += 4096) {
      const int n = min(4096, t1 - tb);
      float mx = -INFINITY;
      for (int i = lane; i < n; i += 64) {
        const uint16_t* kp = seq + (long long)(tb + i) * ldk;
        float acc = 0.f;
        for (int d = 0; d < DQ; d += 8) {
          const U4 kv = ldg16(kp + d);
          acc = fmaf(qs[d + 0], bf16lo(kv.x), acc);
          acc = fmaf(qs[d + 1], bf16hi(kv.x), acc);
          acc = fmaf(qs[d + 2], bf16lo(kv.y), acc);
          acc = fmaf(qs[d + 3], bf16hi(kv.y), acc);
          acc = fmaf(qs[d + 4], bf16lo(kv.z), acc);
          acc = fmaf(qs[d + 5], bf16hi(kv.z), acc);
          acc = fmaf(qs[d + 6], bf16lo(kv.w), acc);
          acc = fmaf(qs[d + 7], bf16hi(kv.w), acc);
        }
        acc *= a.scale_log2;
        sc[i] = acc;
        mx = fmaxf(mx, acc);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float mn = fmaxf(mr, mx);
      const float al = mr == -INFINITY ? 0.f : fast_exp2(mr - mn);
      lr *= al;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] *= al;
      mr = mn;
      for (int i = 0; i < n; ++i) {
        const float pw = fast_exp2(sc[i] - mr);
        lr += pw;
        const uint2 vv = *reinterpret_cast<const uint2*>(seq + (long long)(tb + i) * ldk + r * (DV / 2) + 4 * lane);
        o4[0] = fmaf(pw, bf16lo(vv.x), o4[0]);
        o4[1] = fmaf(pw, bf16hi(vv.x), o4[1]);
        o4[2] = fmaf(pw, bf16lo(vv.y), o4[2]);
        o4[3] = fmaf(pw, bf16hi(vv.y), o4[3]);
      }
    }
    const float inv = 1.f / lr;
    const long long sl = part_slot(a, b, hc, s);
    uint16_t* op = (a.nsplit == 1 ? a.out + ((long long)b * a.Nh + hc) * DV : a.part_o + sl * DV) + r * (DV / 2) + 4 * lane;
    *reinterpret_cast<uint2*>(op) = make_uint2(pack_bf16x2(o4[0] * inv, o4[1] * inv), pack_bf16x2(o4[2] * inv, o4[3] * inv));
    if (a.nsplit > 1 && (c >> 5) == r && lane == 0) {
      a.part_ml[sl * 2 + 0] = mr;
      a.part_ml[sl * 2 + 1] = lr;
    }
  }
}

hipError_t launch(const DecodeArgs& a, hipStream_t st) {
  const long long n_wg = 8 * (((long long)a.B + 7) / 8) * a.nsplit * (a.Nh / kHeads);
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.rope_theta > 0)
    decode_mla_wide_kernel<true><<<dim3((unsigned)n_wg), dim3(kWaves * 64), 0, st>>>(a);
  else
    decode_mla_wide_kernel<false><<<dim3((unsigned)n_wg), dim3(kWaves * 64), 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace wide

template <int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t st) {
  const long long n_hg = a.Nh / (16 * NW);
  const long long pairs = (long long)a.B * a.nsplit;
  const long long n_wg = ((pairs + 7) / 8) * 8 * n_hg;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.rope_theta > 0)
    decode_mla_kernel<NW, true><<<dim3((unsigned)n_wg), dim3(NW * 64), 0, st>>>(a);
  else
    decode_mla_kernel<NW, false><<<dim3((unsigned)n_wg), dim3(NW * 64), 0, st>>>(a);
  return hipGetLastError();
}
}  // namespace

int mla_waves_per_group(int Nh) { return Nh % 128 == 0 ? 8 : Nh % 64 == 0 ? 4 : Nh % 32 == 0 ? 2 : 1; }
int mla_heads_per_group(int Nh) {
  return Nh % wide::kHeads == 0 ? wide::kHeads : Nh % pair::kHeads == 0 ? pair::kHeads : 16 * mla_waves_per_group(Nh);
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t st) {
  if (a.Nh % wide::kHeads == 0) return wide::launch(a, st);
  if (a.Nh % pair::kHeads == 0) return pair::launch(a, st);
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
