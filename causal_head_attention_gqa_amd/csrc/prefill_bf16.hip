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
//   - K/V tiles of 32 keys go from HBM straight into LDS (global_load_lds_dwordx4, no staging
//     registers) through a ring of three stages, so two tiles load while one is computed; rows are
//     stored as in memory with their 16-byte chunks XOR-swizzled by a permutation of the row
//     index, so the K operand reads (16 B per lane, 32 rows) and the transposing V reads
//     (ds_read_b64_tr_b16: 4 consecutive keys of one dim per lane) spread over the LDS banks;
//     the small tiles (48 KiB of LDS per work-group) and 168 registers per lane let three
//     work-groups share a CU;
//   - tiles past the work-group's last query are never visited and 32-key blocks above a wave's
//     diagonal are skipped ("2.7 Transformer Decoder Block完整解析" §3.3); the element mask is
//     applied only on blocks that cross the diagonal or the sequence end;
//   - online softmax per 32-key block ("Transformer 架构完全深度解析" §十三: running max and sum), with the
//     reference max of each query fixed at its first block with a visible key; a block whose
//     exponentials would overflow that reference takes an exact path (new reference, output and sum
//     rescaled), so ordinary blocks compute no row max at all.
//   - K and V operands are read from LDS through small register rings (four K and two V reads in
//     flight), so the products rarely wait on an LDS read.
// All per-wave control values are scalar (wave-uniform branches); per-lane LDS and global
// offsets are computed once. Grid order: work-group i runs on XCD i % 8; when B * Nh / HPW is a
// multiple of 8, each XCD runs its (sequence, head group) pairs one after the other, q-tiles with
// the most key tiles first, so the work-groups resident on an XCD share one pair's K/V in its L2
// (HBM-side reads 1.8x the algorithmic bytes instead of 6x); otherwise the heaviest q-tiles of all
// pairs go first.
#include <type_traits>

#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kBC = 32;     // keys per tile (one 32x32 score block per wave)
constexpr int kStages = 3;  // LDS ring depth: tiles j+1 and j+2 load while tile j is computed
constexpr float kSlack = 8.f;  // log2 units: margin by which the exact path moves the reference max
constexpr float kOvf = 1.8446744e19f;  // 2^64: sum of a block's exponentials that sends it to the exact path
constexpr int kThreads = 256;

// Physical 16-byte chunk of logical chunk c in tile row `row` (CH chunks per row). The XOR key
// permutes the row's low bits (b3 b2 b1 b0 -> b3 b1 b0 b2), a bijection on 8 and on 16
// consecutive rows (K operand reads: 16 B from each of 8-16 consecutive rows) that also sends the
// 4 consecutive rows of one transposing V read to 4 different 32-byte bank groups.
// Rows of 24 chunks (192-dim keys) use a 3-bit key from row bits 1, 3 and 4, which keeps the 32-row
// K operand reads free of bank conflicts at that 384-byte pitch (gfx950 serves a 128-bit read in
// passes of 16 lanes: lane bit 5 and the parity of lane bits 2-4 select the pass).
template <int CH>
__device__ __forceinline__ int swz(int c, int row) {
  if constexpr (CH == 24) return c ^ (((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 4) & 1) << 2));
  const int key = ((row & 3) << 1) | ((row >> 2) & 1) | (CH == 16 ? (row & 8) : 0);
  return c ^ key;
}

// kCache: queries start at q_start[b] (a chunk against a cache); kWin: sliding window + sinks.
// Both are compile-time switches so that the whole-sequence prefill carries none of their code.
// DQK: head dim of q and k; DV: head dim of v and the output (MLA's non-absorbed prefill has
// DQK = 192, DV = 128, its decoupled RoPE block being the last 64 q/k dims).
template <int DQK, int DV, int HPW, bool kCache, bool kWin>
__global__ __launch_bounds__(kThreads, (DQK > 128 ? 2 : 3)) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, const float2* __restrict__ table, int B, int S, int Nh, int Nkv, float c,
    int causal, int n_ptiles, long long kv_tok, long long kv_batch, int kv_head, const int* __restrict__ q_start,
    int max_keys, int window, int sinks, int rope_dims, int rope_inter, long long v_tok, long long v_batch,
    int v_head, unsigned int* __restrict__ lists) {
  constexpr int BP = 32 * (4 / HPW);        // query positions per work-group
  constexpr int CHK = DQK / 8;              // 16-byte chunks per K row
  constexpr int CHV = DV / 8;               // 16-byte chunks per V row
  constexpr int LPK = kBC * CHK / 64 / 4;   // K load instructions per wave per tile
  constexpr int LPV = kBC * CHV / 64 / 4;   // V load instructions per wave per tile
  constexpr int NQ = DQK / 16;              // MFMA k-steps over the q/k head dim
  constexpr int NDB = DV / 32;              // 32-row blocks of the output's head dim
  constexpr int kRopeOff = DQK == DV ? 0 : DV;  // first rotated q dim: 0, or MLA's decoupled block
  static_assert(kBC * CHK % 256 == 0 && kBC * CHV % 256 == 0, "tile loads must split over 4 waves");

  // one array per ring stage, so the compiler can tell which direct-to-LDS loads a read depends on
  static_assert(kStages == 3, "the ring below is written out for three stages");
  __shared__ __attribute__((aligned(1024))) uint16_t Ks0[kBC * DQK];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs0[kBC * DV];
  __shared__ __attribute__((aligned(1024))) uint16_t Ks1[kBC * DQK];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs1[kBC * DV];
  __shared__ __attribute__((aligned(1024))) uint16_t Ks2[kBC * DQK];
  __shared__ __attribute__((aligned(1024))) uint16_t Vs2[kBC * DV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int HGn = Nh / HPW;
  // Work item: (sequence, head group) pair x q-tile. Work-group id runs on XCD id % 8. When the pairs
  // split evenly over the 8 XCDs, XCD x owns one pair of each block of 8 consecutive pairs, pair
  // 8j + (x + j) % 8 of block j, and its list of items goes q-tile-major, heaviest first across those
  // pairs: its resident work-groups share a few pairs' K/V in its L2, and its last work-groups are
  // light ones (taking its pairs one after another instead left the last pair's heavy q-tiles running
  // alone at the end). The rotation by j gives an XCD different KV heads of different sequences (pair
  // x of every block would be KV head x of every sequence: one 256-byte slice of every cache row,
  // which made those XCDs measurably slower than the others). Otherwise the heaviest q-tiles of all
  // pairs go first.
  // Without counters (lists == nullptr) item i of list x is work-group 8i + x. The XCDs run at
  // different clocks, though, and a fixed share leaves the fast ones idle at the end; with counters
  // (8, 64 bytes apart, zeroed before the launch; the grid has an eighth more work-groups than
  // items) a work-group claims the next item of its XCD's list and, once that is used up, of the
  // first list (in rotation order from its own) that still has items; with none left it exits.
  const int npairs = B * HGn;
  int bh, pt;
  if (npairs % 8 == 0) {
    const int ppx = npairs / 8;  // pairs per XCD
    const int per_x = ppx * n_ptiles;
    int x = (int)(blockIdx.x % 8u), c = (int)(blockIdx.x / 8u);
    if (lists != nullptr) {
      __shared__ int s_item;
      if (w == 0) {
        int it = -1;
        unsigned int c0 = 0;
        if (lane == 0) c0 = atomicAdd(&lists[x * 16], 1u);
        c0 = __shfl(c0, 0);
        if (c0 < (unsigned int)per_x) it = x * per_x + (int)c0;
        // every failed claim finds one more list used up, so 8 rounds bound the search
        for (int round = 0; it < 0 && round < 8; ++round) {
          const unsigned int used =
              lane < 8 ? __hip_atomic_load(&lists[lane * 16], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
          const unsigned long long open = __ballot(lane < 8 && used < (unsigned int)per_x);
          if (open == 0) break;
          const unsigned long long rot = ((open >> x) | (open << (8 - x))) & 0xffull;  // bit k: list (x+k)%8
          const int xk = (x + __builtin_ctzll(rot)) & 7;
          unsigned int ck = 0;
          if (lane == 0) ck = atomicAdd(&lists[xk * 16], 1u);
          ck = __shfl(ck, 0);
          if (ck < (unsigned int)per_x) it = xk * per_x + (int)ck;
        }
        if (lane == 0) s_item = it;
      }
      __syncthreads();
      const int it = s_item;
      if (it < 0) return;  // every list used up (the whole work-group leaves)
      x = it / per_x;
      c = it % per_x;
    }
    const int j = c % ppx;
    bh = 8 * j + (x + j) % 8;
    pt = n_ptiles - 1 - c / ppx;
  } else {
    const int id = blockIdx.x;
    bh = id % npairs;
    pt = n_ptiles - 1 - id / npairs;
  }
  const int b = bh / HGn;
  const int h0 = (bh % HGn) * HPW;
  const int g = h0 / (Nh / Nkv);
  const int p0 = pt * BP;
  // queries sit at absolute positions off .. off+S-1 and see keys 0 .. Sk-1 (off = 0: plain prefill;
  // a chunk of a longer sequence otherwise, with the causal mask aligned to the last key)
  const int off = kCache ? min(max(q_start[b], 0), max_keys - S) : 0;
  const int Sk = off + S;
  const int h = h0 + (w % HPW);
  const int wp0 = p0 + (w / HPW) * 32;  // wave's first query position (scalar)
  const int col = lane & 31, hh = lane >> 5;
  const int p = wp0 + col;               // this lane's query position

  // ---- Q^T operand in registers (RoPE applied here when a table is given) ----
  bf16x8 qreg[NQ];
  {
    U4 raw[NQ];
    if (p < S) {
      const uint16_t* qp = q + (((long long)b * S + p) * Nh + h) * DQK + hh * 8;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = ldg16(qp + kk * 16);
      if (table) {
        // rotary span: the leading rope_dims dims (a multiple of 32), table row = rope_dims / 2 pairs
        const float2* tb = table + (long long)(off + p) * (rope_dims / 2);
        if (rope_inter) {  // adjacent pairs (2j, 2j+1): both halves of one 32-bit word
#pragma unroll
          for (int kk = 0; kk < NQ - kRopeOff / 16; ++kk) {
            if (kk * 16 >= rope_dims) break;
            uint32_t* pw = &raw[kRopeOff / 16 + kk].x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float2 cs = tb[kk * 8 + hh * 4 + e];
              const float a = bf16lo(pw[e]), bb = bf16hi(pw[e]);
              pw[e] = pack_bf16x2(fmaf(a, cs.x, -(bb * cs.y)), fmaf(a, cs.y, bb * cs.x));
            }
          }
        } else {  // half-split pairs (i, i + rope_dims/2): registers kk and kk + rope_dims/32
          auto half = [&](auto nr_c) {
            constexpr int NR = decltype(nr_c)::value;
#pragma unroll
            for (int kk = 0; kk < NR; ++kk) {
              uint32_t* pa = &raw[kRopeOff / 16 + kk].x;
              uint32_t* pb = &raw[kRopeOff / 16 + kk + NR].x;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float2 c0 = tb[kk * 16 + hh * 8 + 2 * e], c1 = tb[kk * 16 + hh * 8 + 2 * e + 1];
                const float a0 = bf16lo(pa[e]), a1 = bf16hi(pa[e]);
                const float b0 = bf16lo(pb[e]), b1 = bf16hi(pb[e]);
                pa[e] = pack_bf16x2(fmaf(a0, c0.x, -(b0 * c0.y)), fmaf(a1, c1.x, -(b1 * c1.y)));
                pb[e] = pack_bf16x2(fmaf(a0, c0.y, b0 * c0.x), fmaf(a1, c1.y, b1 * c1.x));
              }
            }
          };
          // one branch per span: rope_dims / 32 register pairs (the host accepts multiples of 32
          // up to the rotated block's width, so every accepted span has its branch)
          if (rope_dims == 32) half(std::integral_constant<int, 1>{});
          else if (rope_dims == 64) half(std::integral_constant<int, 2>{});
          else if constexpr (DQK - kRopeOff >= 96) {
            if (rope_dims == 96) half(std::integral_constant<int, 3>{});
            else if constexpr (DQK - kRopeOff >= 128) {
              if (rope_dims == 128) half(std::integral_constant<int, 4>{});
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = U4{0, 0, 0, 0};
    }
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
    retire_vmem();  // from here on only the tile loads count in vmcnt (they complete in order)
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m = -INFINITY;  // softmax reference max (scale*log2(e) units) of this lane's query
  float mneg = -0.f;     // -m, or 0 while m = -inf: the exponent offset, updated only when m moves
  float lsum = 0.f;     // running sum over the keys this lane holds

  // ---- per-lane global source offsets of the tile loads (row r of a tile, swizzled chunk) ----
  const uint16_t* kbase = k + (long long)b * kv_batch + (long long)g * kv_head;
  const uint16_t* vbase = v + (long long)b * v_batch + (long long)g * v_head;
  // lane i of load instruction sl covers tile bytes sl*1024 + 16*i = row * (row bytes) + 16 * chunk
  // (offsets within one tile stay far below 2^31 elements)
  auto krow = [&](int sl) { return (sl * 1024 + 16 * lane) / (DQK * 2); };
  auto kchk = [&](int sl) { return ((sl * 1024 + 16 * lane) % (DQK * 2)) / 16; };
  auto vrow = [&](int sl) { return (sl * 1024 + 16 * lane) / (DV * 2); };
  auto vchk = [&](int sl) { return ((sl * 1024 + 16 * lane) % (DV * 2)) / 16; };
  int loffk[LPK], loffv[LPV];
#pragma unroll
  for (int r = 0; r < LPK; ++r) {
    const int sl = w * LPK + r;
    loffk[r] = krow(sl) * (int)kv_tok + swz<CHK>(kchk(sl), krow(sl)) * 8;
  }
#pragma unroll
  for (int r = 0; r < LPV; ++r) {
    const int sl = w * LPV + r;
    loffv[r] = vrow(sl) * (int)v_tok + swz<CHV>(vchk(sl), vrow(sl)) * 8;
  }

  // ---- per-lane LDS read offsets (elements), identical for every tile ----
  // K operand: row kb*32 + col, logical chunk 2*kk + hh. For DQK = 64 / 128 the element offset of
  // chunk 2kk + hh is kb_lane ^ (16 kk): the XOR key only changes bits below DQK and col * DQK is a
  // multiple of DQK; 192-dim rows keep one offset per k-step.
  int koff[NQ];
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk) koff[kk] = col * DQK + swz<CHK>(2 * kk + hh, col) * 8;
  const int kb_lane = col * DQK + swz<CHK>(hh, col) * 8;
  auto kaddr = [&](int kk) {
    if constexpr (DQK <= 128) return kb_lane ^ (16 * kk);
    else return koff[kk];
  };
  // V operand (transposing read): rows kb*32 + 16s + 8t + hh*4 + j, dims db*32 + dq*16 + 4c.
  // With row = hh*4 + j (< 8) the swizzle key has bit 3 clear, so the physical chunk of
  // db*4 + x is ((db ^ key>>2) * 4) + (x ^ (key & 3)): only db's parity interacts with the lane,
  // and adding 8 rows (t = 1) flips chunk bit 3, a +-8-chunk shift fixed by db >> 1. Two
  // registers (even / odd db) plus compile-time immediates give every read's address.
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, tr_dq = (lane >> 4) & 1;
  int voff_par[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = hh * 4 + tr_j;
    voff_par[par] = row * DV + swz<CHV>(par * 4 + tr_dq * 2 + (tr_c >> 1), row) * 8 + (tr_c & 1) * 4;
  }
  // element offset of the read for (t, db): voff_par[db & 1] + vimm(t, db)
  auto vimm = [](int t, int db) {
    const int dbase = (db & ~1) * 32;  // chunk (db & ~1)*4 -> element offset, unchanged by keys < 8
    const int tshift = CHV == 16 ? (((db >> 1) & 1) ? -64 : 64) : 0;  // chunk bit 3 flip for rows + 8
    return dbase + t * (8 * DV + tshift);
  };

  const int last = causal ? min(Sk, off + p0 + BP) : Sk;
  const int n_tiles = (last + kBC - 1) / kBC;
  // Key tiles visited: with a sliding window, the sink tiles 0 .. ns-1 and then the tiles from the
  // work-group's earliest window start w0 on; without one, every tile (ns = w0 = 0).
  int ns = 0, w0 = 0;
  if (kWin) {
    w0 = max(off + p0 - window + 1, 0) / kBC;
    ns = min((sinks + kBC - 1) / kBC, w0);
  }
  const int n_vt = ns + (n_tiles - w0);
  auto tile_of = [&](int vt) { return vt < ns ? vt : w0 + (vt - ns); };

  auto issue_tile = [&](int jt, uint16_t* kdst, uint16_t* vdst) {
    if (DQK != DV && jt * kBC + kBC <= Sk) {
      // full tile, 64-bit per-lane addresses (the 192-dim variant keeps its base pointers in
      // vector registers, so the scalar-base form below does not apply)
#pragma unroll
      for (int r = 0; r < LPK; ++r)
        load_lds16_async<false>(kbase + (long long)jt * kBC * kv_tok + loffk[r], kdst + (w * LPK + r) * 512);
#pragma unroll
      for (int r = 0; r < LPV; ++r)
        load_lds16_async<false>(vbase + (long long)jt * kBC * v_tok + loffv[r], vdst + (w * LPV + r) * 512);
    } else if (jt * kBC + kBC <= Sk) {
#pragma unroll
      for (int r = 0; r < LPK; ++r)
        load_lds16_async_sv(kbase + (long long)jt * kBC * kv_tok, 2u * (uint32_t)loffk[r], kdst + (w * LPK + r) * 512);
#pragma unroll
      for (int r = 0; r < LPV; ++r)
        load_lds16_async_sv(vbase + (long long)jt * kBC * v_tok, 2u * (uint32_t)loffv[r], vdst + (w * LPV + r) * 512);
    } else {  // last, partial tile: rows past the end re-read row Sk-1 (finite data, masked)
#pragma unroll
      for (int r = 0; r < LPK; ++r) {
        const int sl = w * LPK + r;
        const int key = min(jt * kBC + krow(sl), Sk - 1);
        load_lds16_async<false>(kbase + (long long)key * kv_tok + swz<CHK>(kchk(sl), krow(sl)) * 8, kdst + sl * 512);
      }
#pragma unroll
      for (int r = 0; r < LPV; ++r) {
        const int sl = w * LPV + r;
        const int key = min(jt * kBC + vrow(sl), Sk - 1);
        load_lds16_async<false>(vbase + (long long)key * v_tok + swz<CHV>(vchk(sl), vrow(sl)) * 8, vdst + sl * 512);
      }
    }
  };

  auto compute_tile = [&](int jt, const uint16_t* Kt, const uint16_t* Vt) {
    const int kb0 = jt * kBC;
    // skip the block when it lies entirely above this wave's diagonal, or entirely before every
    // row's window and past the sinks
    if (causal && kb0 > off + wp0 + 31) return;
    if (kWin && kb0 + 31 < off + wp0 - window + 1 && kb0 >= sinks) return;
    // four K operands in flight: the read of k-step kk + 4 is issued behind the product of kk
    constexpr int R = 4 < NQ ? 4 : NQ;
    bf16x8 ka[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(Kt + kaddr(i));
    f32x16 sv = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      sv = mfma32x32x16(ka[kk % R], qreg[kk], sv);
      if (kk + R < NQ) ka[kk % R] = *reinterpret_cast<const bf16x8*>(Kt + kaddr(kk + R));
    }
    // ---- mask (only on blocks crossing the diagonal or the sequence end) ----
    if ((causal && kb0 + 31 > off + wp0) || kb0 + 32 > Sk || (kWin && kb0 < off + wp0 + 32 - window)) {
      const int base = kb0 + hh * 4;  // key of this lane's score offset 0
      const int hi = (causal ? min(off + p, Sk - 1) : Sk - 1) - base;  // offsets above: after the query
      const int lo = kWin ? off + p - window + 1 - base : -64;  // offsets below: before the window
      const int sk = sinks - base;                                    // offsets below: sinks (kept)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int o = (i >> 2) * 8 + (i & 3);
        if (o > hi || (o < lo && o >= sk)) sv[i] = -INFINITY;
      }
    }
    // Reference max m per query: the max of the row's first block with a visible key (the block
    // max is computed only while some row of the wave has none yet); later blocks exponentiate
    // against it as is, with no per-block max. A score up to ~2^60 above m keeps p, l and O finite
    // (bf16 and fp32 share the exponent range); a block whose exponentials sum past 2^kOvf takes
    // the exact path: its max becomes the reference (when it exceeds m by more than kSlack), O and l
    // are rescaled and the block is exponentiated again. Lanes l and l ^ 32 hold the same query and
    // always agree on m.
    auto block_max = [&]() {
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sv[i]);
      return pair_max32(mt) * c;
    };
    auto set_ref = [&](float mr) {
      m = mr;
      mneg = mr == -INFINITY ? -0.f : -mr;
    };
    if (__builtin_expect(__ballot(m == -INFINITY) != 0, 0)) {
      const float mb = block_max();
      if (m == -INFINITY) set_ref(mb);
    }
    uint32_t pk[2][4];
    float psum;
    auto exps = [&]() {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(fmaf(sv[i], c, mneg));
        const float e1 = fast_exp2(fmaf(sv[i + 1], c, mneg));
        psum = i == 0 ? e0 + e1 : psum + (e0 + e1);
        pk[i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
      }
    };
    exps();
    if (__builtin_expect(__ballot(!(psum <= kOvf)) != 0, 0)) {  // rare: a score far above the reference
      const float mb = block_max();
      const bool move = mb > m + kSlack;  // never for a row without a visible key (then mb = m = -inf)
      const float alpha = move ? fast_exp2(m - mb) : 1.f;
      if (move) set_ref(mb);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      exps();
    }
    lsum += psum;

    // ---- O^T += V^T P^T over this block's 32 keys ----
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, U4{pk[s][0], pk[s][1], pk[s][2], pk[s][3]});
      const uint16_t* Vb = Vt + 16 * s * DV;
      auto vread = [&](int db) {
        const uint2 lo = lds_read_tr16(Vb + voff_par[db & 1] + vimm(0, db));
        const uint2 hi = lds_read_tr16(Vb + voff_par[db & 1] + vimm(1, db));
        return __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      };
      // two V operands in flight (the read of block db + 2 behind the product of db)
      bf16x8 va[2];
      va[0] = vread(0);
      va[1] = vread(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        o[db] = mfma32x32x16(va[db & 1], bop, o[db]);
        if (db + 2 < NDB) va[db & 1] = vread(db + 2);
      }
    }
  };

  // ---- ring of kStages tiles: wait for this wave's loads of tile jt (those of tile jt+1 may
  // fly), then a barrier makes every wave's part of the tile visible. A load past the last tile
  // re-reads the last one into a stage that is never read again, so every step issues the same
  // loads and each wait keeps one fixed count (the compiler's own waits stay exact as well). ----
  issue_tile(tile_of(0), Ks0, Vs0);
  issue_tile(tile_of(min(1, n_vt - 1)), Ks1, Vs1);
  auto step = [&](int jt, const uint16_t* Kt, const uint16_t* Vt, uint16_t* kn, uint16_t* vn) {
    wait_vmem_n<LPK + LPV>();
    barrier_only();
    issue_tile(tile_of(min(jt + 2, n_vt - 1)), kn, vn);
    compute_tile(tile_of(jt), Kt, Vt);
  };
  for (int jt = 0; jt < n_vt; jt += 3) {
    step(jt, Ks0, Vs0, Ks2, Vs2);
    if (jt + 1 >= n_vt) break;
    step(jt + 1, Ks1, Vs1, Ks0, Vs0);
    if (jt + 2 >= n_vt) break;
    step(jt + 2, Ks2, Vs2, Ks1, Vs1);
  }

  wait_vmem();  // the re-read past the last tile must land before the work-group's LDS is released

  // ---- epilogue: O / l, round to bf16, store BSHD ----
  const float inv = 1.f / pair_sum32(lsum);
  if (p < S) {
    uint16_t* op = out + (((long long)b * S + p) * Nh + h) * DV + hh * 4;
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

// Zeroes the work lists' counters of prefill_bf16_kernel before its launch.
__global__ void prefill_lists_reset_kernel(unsigned int* __restrict__ lists) {
  if (threadIdx.x < 8 * 16) lists[threadIdx.x] = 0u;
}

// ---- split-key prefill, for grids too small to fill the chip ----
//
// With few (sequence, head) pairs and a short sequence (GPT-2-small: 96 pairs of 1024 tokens), the
// kernel above has too few work-groups, and its critical path is the wave that holds a sequence's
// last 32 rows: one dependent chain over every key tile. Here the 4 waves of a work-group split
// the key tiles of their query rows KS ways: the work-group holds 4/KS blocks of 32 query rows of
// one head, and wave w takes block w / KS and the key tiles w % KS, w % KS + KS, ... (a KS-th of the
// chain). The waves of one key split (one per query block) need the same tiles, so they share a
// 2-stage LDS ring, each loading its part of every tile (direct-to-LDS loads); one work-group barrier
// per step makes a tile visible and frees the other stage. Each wave runs the online softmax of the
// kernel above on its tiles (fixed reference max, exact path for a block that overflows it); at the
// end the KS partial (max, sum, output) of each block are merged through LDS with the same
// recurrences ("Transformer 架构完全深度解析" §十三: running max and sum, applied to the waves'
// partial results). The shared rings take half the LDS of one ring per wave (35 KiB for 64-dim
// heads), so four work-groups share a CU. Plain prefill only (positions 0 .. S-1, no cache, no
// window), equal q/k/v head dims, half-split RoPE over the whole head when a table is given.
template <int D, int KS>
__global__ __launch_bounds__(kThreads, (D <= 64 ? 4 : 2)) void prefill_splitk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, const float2* __restrict__ table, int B, int S, int Nh, int Nkv, float c, int causal,
    int n_qb) {
  constexpr int NB = 2;                 // stages of each key split's ring
  constexpr int CH = D / 8;             // 16-byte chunks per row
  constexpr int TE = kBC * D;           // elements of one K (or V) tile
  constexpr int LT = kBC * CH / 64;     // load instructions per K (or V) tile, one wave
  constexpr int NQ = D / 16;            // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;           // 32-row blocks of the output's head dim
  constexpr int MP = D + 4;             // row pitch (floats) of the merge area
  constexpr int QB = 4 / KS;            // 32-row query blocks per work-group
  constexpr int LW = LT / QB;           // load instructions per K (or V) tile and wave of a ring
  static_assert(LT % QB == 0, "a ring's tile loads split evenly over its waves");
  // the KS rings [KS][NB][K, V][TE], then (once the loop is done) the merge area of each wave
  constexpr int kRingBytes = KS * NB * 2 * TE * 2;
  constexpr int kMergeFloats = 32 * MP + 64;  // one wave's rows, then its (max, sum) pairs
  constexpr int kLdsBytes = kRingBytes > 4 * kMergeFloats * 4 ? kRingBytes : 4 * kMergeFloats * 4;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kLdsBytes / 2];
  auto ring = [&](int ksr, int st, int kv) { return lds + ((ksr * NB + st) * 2 + kv) * TE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // heaviest blocks first, (sequence, head) fastest; n_qb counts groups of QB blocks
  const int nbh = B * Nh;
  const int id = blockIdx.x;
  const int bh = id % nbh;
  const int qg = n_qb - 1 - id / nbh;
  const int b = bh / Nh, h = bh % Nh;
  const int g = h / (Nh / Nkv);
  const int qsub = w / KS, ks = w % KS;  // the wave's query block within the group, its key split
  const int p0 = (qg * QB + qsub) * 32;
  const int col = lane & 31, hh = lane >> 5;
  const int p = p0 + col;  // this lane's query position

  // ---- Q^T operand (RoPE at position p when a table is given) ----
  bf16x8 qreg[NQ];
  {
    U4 raw[NQ];
    if (p < S) {
      const uint16_t* qp = q + (((long long)b * S + p) * Nh + h) * D + hh * 8;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = ldg16(qp + kk * 16);
      if (table) {  // half-split pairs (i, i + D/2): registers kk and kk + NQ/2
        const float2* tb = table + (long long)p * (D / 2);
#pragma unroll
        for (int kk = 0; kk < NQ / 2; ++kk) {
          uint32_t* pa = &raw[kk].x;
          uint32_t* pb = &raw[kk + NQ / 2].x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float2 c0 = tb[kk * 16 + hh * 8 + 2 * e], c1 = tb[kk * 16 + hh * 8 + 2 * e + 1];
            const float a0 = bf16lo(pa[e]), a1 = bf16hi(pa[e]);
            const float b0 = bf16lo(pb[e]), b1 = bf16hi(pb[e]);
            pa[e] = pack_bf16x2(fmaf(a0, c0.x, -(b0 * c0.y)), fmaf(a1, c1.x, -(b1 * c1.y)));
            pb[e] = pack_bf16x2(fmaf(a0, c0.y, b0 * c0.x), fmaf(a1, c1.y, b1 * c1.x));
          }
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) raw[kk] = U4{0, 0, 0, 0};
    }
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
    retire_vmem();  // from here on only the tile loads count in vmcnt
  }

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m = -INFINITY, mneg = -0.f, lsum = 0.f;

  // ---- key tiles needed by query block qs of this work-group (none past the sequence); the
  // work-group's largest need sets the step count, the same for every wave ----
  auto need = [&](int qs) {
    const int pq = (qg * QB + qs) * 32;
    return pq >= S ? 0 : ((causal ? min(S, pq + 32) : S) + kBC - 1) / kBC;
  };
  int max_tiles = 0;
#pragma unroll
  for (int qs = 0; qs < QB; ++qs) max_tiles = max(max_tiles, need(qs));
  const int n_steps = (max_tiles + KS - 1) / KS;  // tiles of key split 0, the most of any split
  const int my_tiles = need(qsub);
  const long long kv_tok = (long long)Nkv * D;
  const uint16_t* kbase = k + (long long)b * S * kv_tok + (long long)g * D;
  const uint16_t* vbase = v + (long long)b * S * kv_tok + (long long)g * D;
  // lane i of load sl covers tile bytes sl*1024 + 16i = row * 2D + 16 * chunk
  auto trow = [&](int sl) { return (sl * 1024 + 16 * lane) / (D * 2); };
  auto tchk = [&](int sl) { return ((sl * 1024 + 16 * lane) % (D * 2)) / 16; };
  // this wave loads slots qsub * LW .. qsub * LW + LW - 1 of every K and V tile of its ring
  uint32_t loff[LW];
#pragma unroll
  for (int u = 0; u < LW; ++u) {
    const int sl = qsub * LW + u;
    loff[u] = 2u * (uint32_t)(trow(sl) * (int)kv_tok + swz<CH>(tchk(sl), trow(sl)) * 8);
  }
  auto issue_tile = [&](int jt, uint16_t* kdst, uint16_t* vdst) {
    if (jt * kBC + kBC <= S) {
      asm volatile("s_nop 4" ::: "memory");
#pragma unroll
      for (int u = 0; u < LW; ++u)
        load_lds16_async_sv(kbase + (long long)jt * kBC * kv_tok, loff[u], kdst + (qsub * LW + u) * 512);
#pragma unroll
      for (int u = 0; u < LW; ++u)
        load_lds16_async_sv(vbase + (long long)jt * kBC * kv_tok, loff[u], vdst + (qsub * LW + u) * 512);
    } else {  // the last, partial tile: rows past the end re-read row S-1 (finite data, masked)
#pragma unroll
      for (int u = 0; u < LW; ++u) {
        const int sl = qsub * LW + u;
        const long long e = (long long)min(jt * kBC + trow(sl), S - 1) * kv_tok + swz<CH>(tchk(sl), trow(sl)) * 8;
        load_lds16_async<false>(kbase + e, kdst + sl * 512);
        load_lds16_async<false>(vbase + e, vdst + sl * 512);
      }
    }
  };

  // ---- per-lane LDS read offsets: as in the kernel above ----
  const int kb_lane = col * D + swz<CH>(hh, col) * 8;
  const int tr_j = (lane & 15) >> 2, tr_c = lane & 3, tr_dq = (lane >> 4) & 1;
  int voff_par[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int row = hh * 4 + tr_j;
    voff_par[par] = row * D + swz<CH>(par * 4 + tr_dq * 2 + (tr_c >> 1), row) * 8 + (tr_c & 1) * 4;
  }
  auto vimm = [](int t, int db) {
    const int dbase = (db & ~1) * 32;
    const int tshift = CH == 16 ? (((db >> 1) & 1) ? -64 : 64) : 0;
    return dbase + t * (8 * D + tshift);
  };

  auto compute_tile = [&](int jt, const uint16_t* Kt, const uint16_t* Vt) {
    const int kb0 = jt * kBC;
    constexpr int R = 4 < NQ ? 4 : NQ;
    bf16x8 ka[R];
#pragma unroll
    for (int i = 0; i < R; ++i) ka[i] = *reinterpret_cast<const bf16x8*>(Kt + (kb_lane ^ (16 * i)));
    f32x16 sv = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      sv = mfma32x32x16(ka[kk % R], qreg[kk], sv);
      if (kk + R < NQ) ka[kk % R] = *reinterpret_cast<const bf16x8*>(Kt + (kb_lane ^ (16 * (kk + R))));
    }
    if ((causal && kb0 + 31 > p0) || kb0 + 32 > S) {  // the diagonal block or the sequence end
      const int base = kb0 + hh * 4;
      const int hi = (causal ? min(p, S - 1) : S - 1) - base;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i >> 2) * 8 + (i & 3) > hi) sv[i] = -INFINITY;
    }
    auto block_max = [&]() {
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sv[i]);
      return pair_max32(mt) * c;
    };
    auto set_ref = [&](float mr) {
      m = mr;
      mneg = mr == -INFINITY ? -0.f : -mr;
    };
    if (__builtin_expect(__ballot(m == -INFINITY) != 0, 0)) {
      const float mb = block_max();
      if (m == -INFINITY) set_ref(mb);
    }
    uint32_t pk[2][4];
    float psum;
    auto exps = [&]() {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float e0 = fast_exp2(fmaf(sv[i], c, mneg));
        const float e1 = fast_exp2(fmaf(sv[i + 1], c, mneg));
        psum = i == 0 ? e0 + e1 : psum + (e0 + e1);
        pk[i >> 3][(i & 7) >> 1] = pack_bf16x2(e0, e1);
      }
    };
    exps();
    if (__builtin_expect(__ballot(!(psum <= kOvf)) != 0, 0)) {  // rare: a score far above the reference
      const float mb = block_max();
      const bool move = mb > m + kSlack;
      const float alpha = move ? fast_exp2(m - mb) : 1.f;
      if (move) set_ref(mb);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      exps();
    }
    lsum += psum;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bf16x8 bop = __builtin_bit_cast(bf16x8, U4{pk[s2][0], pk[s2][1], pk[s2][2], pk[s2][3]});
      const uint16_t* Vb = Vt + 16 * s2 * D;
      auto vread = [&](int db) {
        const uint2 lo = lds_read_tr16(Vb + voff_par[db & 1] + vimm(0, db));
        const uint2 hi = lds_read_tr16(Vb + voff_par[db & 1] + vimm(1, db));
        return __builtin_bit_cast(bf16x8, U4{lo.x, lo.y, hi.x, hi.y});
      };
      bf16x8 va[2];
      va[0] = vread(0);
      if (NDB > 1) va[1] = vread(1);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        o[db] = mfma32x32x16(va[db & 1], bop, o[db]);
        if (db + 2 < NDB) va[db & 1] = vread(db + 2);
      }
    }
  };

  // ---- step i: tile ks + KS*i of every key split. Each wave waits for its own part of the tile,
  // the barrier makes the whole tile visible and guarantees that every wave is done with the other
  // stage (the tile of step i-1), which the loads of step i+1 then refill. Every wave runs all
  // n_steps steps (the barrier count is the work-group's), computing only the tiles its block
  // needs; a ring holds every tile that either of its blocks needs. ----
  auto issue_step = [&](int i) {
    const int jt = ks + KS * i;
    if (jt < max_tiles) issue_tile(jt, ring(ks, i & 1, 0), ring(ks, i & 1, 1));
  };
  issue_step(0);
  for (int i = 0; i < n_steps; ++i) {
    wait_vmem_n<0>();  // this wave's part of step i's tile has landed (nothing newer is in flight)
    barrier_only();
    issue_step(i + 1);
    const int jt = ks + KS * i;
    if (jt < my_tiles) compute_tile(jt, ring(ks, i & 1, 0), ring(ks, i & 1, 1));
  }
  __syncthreads();  // every wave is done with the rings: the merge area overlays them

  // ---- merge the KS waves of each block: (max, sum, output) through LDS ----
  auto mo = [&](int vw) { return reinterpret_cast<float*>(lds) + vw * kMergeFloats; };
  const float ltot = pair_sum32(lsum);
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4*>(mo(w) + col * MP + db * 32 + g4 * 8 + hh * 4) =
          f32x4{o[db][g4 * 4], o[db][g4 * 4 + 1], o[db][g4 * 4 + 2], o[db][g4 * 4 + 3]};
  if (hh == 0) {
    mo(w)[32 * MP + col * 2] = m;  // -inf for a wave without tiles (its sum and output are 0)
    mo(w)[32 * MP + col * 2 + 1] = ltot;
  }
  __syncthreads();
  // thread t: row r = t / (8 / QB) of the group's 32 * QB rows, D / (8 / QB) dims from d0
  constexpr int TPR = 8 / QB;   // threads per query row
  constexpr int PER = D / TPR;  // output dims per thread
  const int r = tid / TPR, qq = r % 32, w0 = (r / 32) * KS, d0 = (tid % TPR) * PER;
  const int pr = (qg * QB + r / 32) * 32 + qq;  // the row's position
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < KS; ++u) mx = fmaxf(mx, mo(w0 + u)[32 * MP + qq * 2]);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const float mv = mo(w0 + u)[32 * MP + qq * 2];
    const float wgt = mv == -INFINITY ? 0.f : fast_exp2(mv - mx);
    l = fmaf(wgt, mo(w0 + u)[32 * MP + qq * 2 + 1], l);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(wgt, mo(w0 + u)[qq * MP + d0 + e], acc[e]);
  }
  if (pr < S) {
    const float inv = 1.f / l;
    uint16_t* op = out + (((long long)b * S + pr) * Nh + h) * D + d0;
#pragma unroll
    for (int e = 0; e < PER; e += 8)
      stg16(op + e, U4{pack_bf16x2(acc[e] * inv, acc[e + 1] * inv), pack_bf16x2(acc[e + 2] * inv, acc[e + 3] * inv),
                       pack_bf16x2(acc[e + 4] * inv, acc[e + 5] * inv), pack_bf16x2(acc[e + 6] * inv, acc[e + 7] * inv)});
  }
}

// The plain prefill takes the split-key kernel when the usual grid is under two rounds of the
// chip's work-group slots (3 per CU x 256) and the rows are long enough (S >= 512) for one wave's
// chain over every key tile to dominate. Two key splits (two 32-row blocks per work-group): on the
// GPT-2-small shape (96 heads x 1024 tokens) 30.8-31.2 us against 33.7-34.3 us for the kernel above;
// four splits were slower (38 us: twice the work-groups, each paying its prologue and merge), and
// one split (private rings only) equal to two; two splits also halve the chain of long sequences
// with few heads.
constexpr long long kSplitMaxWG = 2 * 3 * 256;
constexpr int kSplitMinS = 512;

constexpr int kSplitKS = 2;  // key splits per query block (4 waves: 4 / KS blocks per work-group)

template <int D>
hipError_t launch_splitk(const PrefillArgs& a, hipStream_t st) {
  constexpr int QB = 4 / kSplitKS;
  const int n_qb = (a.S + 32 * QB - 1) / (32 * QB);  // groups of QB blocks of 32 rows
  const long long n_wg = (long long)n_qb * a.B * a.Nh;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  prefill_splitk_kernel<D, kSplitKS><<<dim3((unsigned)n_wg), dim3(kThreads), 0, st>>>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
      static_cast<uint16_t*>(a.out), a.table, a.B, a.S, a.Nh, a.Nkv, a.scale_log2, a.causal, n_qb);
  return hipGetLastError();
}

template <int DQK, int DV, int HPW, bool kCache, bool kWin>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int BP = 32 * (4 / HPW);
  const int n_ptiles = (a.S + BP - 1) / BP;
  const long long npairs = (long long)a.B * (a.Nh / HPW);
  const long long n_items = (long long)n_ptiles * npairs;
  // with the work lists (pairs split evenly over the XCDs): an eighth more work-groups, which the
  // fast XCDs use to take items from the slow ones' lists
  unsigned int* lists = npairs % 8 == 0 ? a.queue : nullptr;
  const long long n_wg = lists != nullptr ? n_items + 8 * ((n_items / 8 + 7) / 8) : n_items;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (lists != nullptr && !a.queue_zeroed) prefill_lists_reset_kernel<<<dim3(1), dim3(128), 0, st>>>(lists);
  prefill_bf16_kernel<DQK, DV, HPW, kCache, kWin><<<dim3((unsigned)n_wg), dim3(kThreads), 0, st>>>(
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
      static_cast<uint16_t*>(a.out), a.table, a.B, a.S, a.Nh, a.Nkv, a.scale_log2, a.causal, n_ptiles, a.kv_tok,
      a.kv_batch, a.kv_head, a.q_start, a.max_keys, a.window, a.sinks, a.rope_dims, a.rope_inter, a.v_tok, a.v_batch,
      a.v_head, lists);
  return hipGetLastError();
}

template <int DQK, int DV, int HPW>
hipError_t launch_m(const PrefillArgs& a, hipStream_t st) {
  if constexpr (DQK == DV) {
    if (a.window > 0) return launch_t<DQK, DV, HPW, true, true>(a, st);  // windows come through the cache entry
    if (a.q_start) return launch_t<DQK, DV, HPW, true, false>(a, st);
  }
  return launch_t<DQK, DV, HPW, false, false>(a, st);
}

template <int DQK, int DV>
hipError_t launch_d(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Nh / a.Nkv;
  if (G % 4 == 0) return launch_m<DQK, DV, 4>(a, st);
  if (G % 2 == 0) return launch_m<DQK, DV, 2>(a, st);
  return launch_m<DQK, DV, 1>(a, st);
}
}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t st) {
  if (a.Dv != a.D) return a.D == 192 && a.Dv == 128 ? launch_d<192, 128>(a, st) : hipErrorInvalidValue;
  if (!a.q_start && a.window == 0 && a.S >= kSplitMinS && (a.D == 64 || a.D == 128) &&
      (a.table == nullptr || (a.rope_dims == a.D && !a.rope_inter))) {
    const int G = a.Nh / a.Nkv;
    const int hpw = G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1;
    const long long n_wg = (long long)((a.S + 32 * (4 / hpw) - 1) / (32 * (4 / hpw))) * a.B * (a.Nh / hpw);
    if (n_wg < kSplitMaxWG) return a.D == 64 ? launch_splitk<64>(a, st) : launch_splitk<128>(a, st);
  }
  switch (a.D) {
    case 64:
      return launch_d<64, 64>(a, st);
    case 128:
      return launch_d<128, 128>(a, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace attn
