// KV-cache decode for MHA/GQA/MQA on gfx950, split over the context ("split-KV"), plus the
// reduction that merges the splits.
//
// What is computed: for each sequence b and query head h, the single new query attends to the
// cached keys 0 .. ctx_b-1 of KV head h / (Nh/Nkv) with no mask ("Transformer 架构完全深度解析"
// §九: the new K/V are appended first; "Transformer 架构快速入门" §13.2).
//
// Decode streams the cache once at ~4 FLOP per byte, so it is bound by HBM bandwidth. The design
// keeps many bytes in flight and the vector ALUs nearly idle:
//   - a work-group owns (b, one KV head, up to 16 of its query heads, one context chunk): every
//     cached row is fetched once, shared by the query heads of its group in registers;
//   - each of the 4 waves streams its own 16-token stages through a private LDS ring with
//     direct-to-LDS loads (several stages in flight per wave, no barrier while streaming);
//   - the tiny contractions run on the matrix cores with the heads padded to 16 (q.k as
//     16x16x32, p.v as 16x16x16 whose p operand is the score block's own register layout);
//   - each chunk writes its (max, sum) in fp32 and its output normalised by that sum in bf16;
//     the reduction kernel merges
//     the chunks with the online-softmax algebra ("Transformer 架构完全深度解析" §十三: the
//     running max / sum recurrences, applied to whole chunks).
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kThreads = 256;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

// XOR key of the 16-byte chunk index in stage row `row` (CH chunks per row). gfx950 serves a
// 128-bit LDS read in four passes of 16 lanes (equal lane bit 5 and equal parity of lane bits 2-4)
// and a 64-bit read in two passes of 32 lanes; these keys make the K operand reads (16 rows, one
// chunk per 16-lane row group) and the transposing V reads (8 rows x 32 bytes per pass) touch 16
// distinct 16-byte bank groups per pass, i.e. no bank conflicts.
template <int CH>
__device__ __forceinline__ int dkey(int row) {
  return CH == 16 ? ((row & 7) << 1) : (row & 6);
}

// Max / sum over the four 16-lane rows that hold one head's tokens.
__device__ __forceinline__ float rows_max4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max32(fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Chunks of a context: n = ceil(ctx / chunk) of ceil(ctx / n) tokens each (the last one up to n - 1
// tokens shorter): a context of 1025 tokens is two chunks of 513 and 512 tokens, not 1024 and 1.
// The chunk count (and so the merge) is that of fixed chunks; all chunks hold chunk/2 .. chunk tokens.
__device__ __forceinline__ void chunk_plan(int ctx, int chunk, int& n, int& len) {
  n = (ctx + chunk - 1) / chunk;
  len = n > 0 ? (ctx + n - 1) / n : 0;
}

// Work item `item` of the split kernel, in the order the work-groups are dispatched: sequence-major,
// the chunks of a sequence together. With fixed chunks the random-length last chunks formed a round
// of their own after the full ones (every slot finishing its last full chunk at the same time, then
// one short chunk each, ending 0 .. 1 chunk apart); with balanced chunks the lengths are spread over
// the whole grid: -1.7 % split-kernel time in a same-box A/B (a second ordering by length class
// gained no more). Returns false past the last item. Called by every lane of a wave with the same
// `item`; the result is uniform over it.
__device__ __forceinline__ bool decode_item(const DecodeArgs& a, int item, int& b_out, int& s_out) {
  const int lane = threadIdx.x & 63;
  int before = 0;  // chunks of the sequences before this block of 64
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    const int ctx = b < a.B ? min(max(a.ctx_lens[b], 0), a.max_ctx) : 0;
    int f, len;
    chunk_plan(ctx, a.chunk, f, len);
    int incl = f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (item < before + total) {
      const int l = __builtin_ctzll(__ballot(before + incl > item));
      b_out = b0 + l;
      s_out = item - before - (__shfl(incl, l) - __shfl(f, l));
      return true;
    }
    before += total;
  }
  return false;
}

// One work-group = 4 waves for (sequence b, KV head g, up to 16 of its query heads, one chunk).
// Each wave streams its own 16-token stages (stage k of the chunk goes to wave k % 4) through a
// private NB-deep LDS ring filled by direct-to-LDS loads, so no barrier is needed while streaming:
//   S^T[16 tokens x 16 heads] = K Q^T   (v_mfma_f32_16x16x32_bf16, query heads padded to 16)
//   online softmax per head (running max and sum, output rescaled only when some max moved)
//   O^T[D x 16 heads] += V^T P^T        (v_mfma_f32_16x16x16bf16_1k; P^T is the score block's
//                                        own register layout, V^T comes from the transposing read)
// The four waves' (max, sum, output) are merged in LDS and written as the chunk's partial.
template <int D, int NB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int ROWS = 16;           // tokens per stage
  constexpr int SE = ROWS * D;       // elements per stage and operand
  constexpr int LPS = SE * 2 / 1024; // 1 KiB load instructions per stage and operand
  constexpr int NKK = D / 32;        // Q.K k-steps
  constexpr int NDB = D / 16;        // output dim blocks
  __shared__ __attribute__((aligned(1024))) uint16_t ring[4][NB][2][SE];
  static_assert(NB * 2 * SE * 2 >= (16 * (D + 4) + 32) * 4, "merge area must fit in a wave's ring");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Nh / a.Nkv;
  const int HG = G < 16 ? G : 16;
  const int n_hg = G / HG;  // head groups per KV head
  // block order: head group fastest, then the work item (sequence-major, balanced chunks). The KV
  // heads of one token sit side by side in a cache row, so consecutive work-groups (dispatched to
  // different XCDs at the same time) read the neighbouring segments of the same rows together:
  // +12 % bandwidth over a chunk-fastest order, which fetched each head's 256-byte segments of a
  // row at different times. The head group is rotated by the sequence
  // index, so that a work-group id's XCD (id % 8) reads different KV heads of different sequences:
  // with one KV head per XCD (each reading one fixed 256-byte slice of every row) some XCDs ran
  // ~15 % longer than others on the same work.
  const int nhg = a.Nkv * n_hg;
  int b, s;
  if (!decode_item(a, blockIdx.x / nhg, b, s)) return;  // past the last item
  const int hgi = (int)((blockIdx.x + (unsigned)b) % (unsigned)nhg);
  const int g = hgi / n_hg;
  const int h0 = g * G + (hgi % n_hg) * HG;
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  int n_ch, len;
  chunk_plan(ctx, a.chunk, n_ch, len);
  const int t0 = s * len;
  if (t0 >= ctx) return;  // empty split: the reduction ignores it
  const int t1 = min(ctx, t0 + len);
  const int hc = lane & 15, rg = lane >> 4;
  const bool real = hc < HG;

  // ---- Q^T operand (head column hc, dims kk*32 + rg*8 .. +7), rotated at ctx-1 if asked ----
  bf16x8 qreg[NKK];
  {
    U4 raw[NKK];
    const uint16_t* qp = a.q + ((long long)b * a.Nh + h0 + (real ? hc : 0)) * D + rg * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) raw[kk] = real ? ldg16(qp + kk * 32) : U4{0, 0, 0, 0};
    if (a.rope_theta > 0) {
      // one position for every head: lane l evaluates the angle of frequency l % (D/2) once (fp64),
      // the pairs fetch theirs from the lane that holds it (every lane takes part; the padding
      // lanes rotate zeros)
      const double k2 = -2.0 * log2(a.rope_theta) / (double)D;
      double sn_l, cs_l;
      sincos((double)(ctx - 1) * exp2(k2 * (double)(lane % (D / 2))), &sn_l, &cs_l);
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk) {
        uint32_t* pa = &raw[kk].x;
        uint32_t* pb = &raw[kk + NKK / 2].x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float ra[2], rb[2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int i = kk * 32 + rg * 8 + 2 * e + hf;  // pair (i, i + D/2)
            const double sn = __shfl(sn_l, i), cs = __shfl(cs_l, i);
            const double x = hf ? bf16hi(pa[e]) : bf16lo(pa[e]);
            const double y = hf ? bf16hi(pb[e]) : bf16lo(pb[e]);
            ra[hf] = (float)(x * cs - y * sn);
            rb[hf] = (float)(x * sn + y * cs);
          }
          pa[e] = pack_bf16x2(ra[0], ra[1]);
          pb[e] = pack_bf16x2(rb[0], rb[1]);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qreg[kk] = as_bf16x8(raw[kk]);
    retire_vmem();
  }

  // ---- per-lane LDS offsets within a stage (elements) ----
  int koff[NKK];  // K operand: row hc, logical chunk 4*kk + rg
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = hc * D + ((4 * kk + rg) ^ dkey<CH>(hc)) * 8;
  const int tj = (lane & 15) >> 2, tc = lane & 3;
  const int vrow = rg * 4 + tj;  // V operand: rows rg*4 + j, dims db*16 + 4c
  const int vkey = dkey<CH>(vrow);

  // ---- stage loads (this wave only): lane i of instruction r covers stage bytes r*1024 + 16*i ----
  const long long rk = (long long)a.Nkv * a.ldk, rv = (long long)a.Nkv * a.ldv;
  const uint16_t* kb = a.kc + ((long long)b * a.max_ctx * a.Nkv + g) * a.ldk;
  const uint16_t* vb = a.vc + ((long long)b * a.max_ctx * a.Nkv + g) * a.ldv;
  auto issue_stage = [&](int k, int slot) {
    const int tb = t0 + k * ROWS;
#pragma unroll
    for (int r = 0; r < LPS; ++r) {
      const int ob = r * 1024 + 16 * lane;
      const int row = ob / (D * 2);
      const int pc = (ob % (D * 2)) / 16;
      const int t = min(tb + row, t1 - 1);  // rows past the chunk re-read a valid row (masked)
      const int lc = pc ^ dkey<CH>(row);
      load_lds16_async(kb + t * rk + lc * 8, &ring[w][slot][0][r * 512]);
      load_lds16_async(vb + t * rv + lc * 8, &ring[w][slot][1][r * 512]);
    }
  };

  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4{};
  float m = -INFINITY, lsum = 0.f;

  const int n_stages = (t1 - t0 + ROWS - 1) / ROWS;
  const int my_n = n_stages > w ? (n_stages - w + 3) / 4 : 0;  // stages w, w+4, ...
#pragma unroll
  for (int i = 0; i < NB - 1; ++i)
    if (i < my_n) issue_stage(w + 4 * i, i);
  for (int i = 0; i < my_n; ++i) {
    const int k = w + 4 * i;
    const int later = min(my_n - 1 - i, NB - 2);  // stages already issued after this one
    if (later >= 2)
      wait_vmem_n<4 * LPS>();
    else if (later == 1)
      wait_vmem_n<2 * LPS>();
    else
      wait_vmem();
    if (i + NB - 1 < my_n) issue_stage(k + 4 * (NB - 1), (i + NB - 1) % NB);
    const uint16_t* Ks = ring[w][i % NB][0];
    const uint16_t* Vs = ring[w][i % NB][1];

    f32x4 sacc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(Ks + koff[0]), qreg[0], f32x4{});
#pragma unroll
    for (int kk = 1; kk < NKK; ++kk)
      sacc = mfma16x16x32(*reinterpret_cast<const bf16x8*>(Ks + koff[kk]), qreg[kk], sacc);
    const int tb = t0 + k * ROWS + rg * 4;  // tokens of this lane's 4 scores
    if (t0 + k * ROWS + ROWS > t1) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tb + e >= t1) sacc[e] = -INFINITY;
    }
    float mt = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    mt = rows_max4(mt);
    // lazy reference max (moves only when a head's max grows by more than 2^8; see prefill)
    const float mb = mt * a.scale_log2;
    const bool move = mb > m + 8.f;
    const float m_new = move ? mb : m;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = move ? fast_exp2(m - m_use) : 1.f;
    m = m_new;
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(fmaf(sacc[e], a.scale_log2, -m_use));
    lsum = fmaf(lsum, alpha, (pe[0] + pe[1]) + (pe[2] + pe[3]));
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[db][e] *= alpha;
    }
    const i16x4 pb = __builtin_bit_cast(i16x4, make_uint2(pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3])));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int lc = 2 * db + (tc >> 1);
      const uint2 v = lds_read_tr16(Vs + vrow * D + (lc ^ vkey) * 8 + (tc & 1) * 4);
      o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, v), pb, o[db], 0, 0, 0);
    }
  }

  // ---- merge the four waves (per head: max, sum and output), write the chunk partial ----
  const float lt = [&] {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    return pair_sum32(__uint_as_float(r[0]) + __uint_as_float(r[1]));
  }();
  // the merge reuses each wave's own ring area (its loads have all landed): [16][D+4] outputs, then
  // [16][2] (max, sum)
  auto mo = [&](int v) { return reinterpret_cast<float*>(&ring[v][0][0][0]); };
  auto mm = [&](int v) { return reinterpret_cast<float*>(&ring[v][0][0][0]) + 16 * (D + 4); };
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo(w)[hc * (D + 4) + db * 16 + rg * 4 + e] = o[db][e];
  if (rg == 0) {
    mm(w)[hc * 2 + 0] = my_n > 0 ? m : -INFINITY;
    mm(w)[hc * 2 + 1] = my_n > 0 ? lt : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < HG * D; i += kThreads) {
    const int hl = i / D, d = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, mm(v)[hl * 2]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float mv = mm(v)[hl * 2];
      const float wgt = mv == -INFINITY ? 0.f : fast_exp2(mv - mx);
      acc = fmaf(wgt, mo(v)[hl * (D + 4) + d], acc);
      l = fmaf(wgt, mm(v)[hl * 2 + 1], l);
    }
    const long long slot = part_slot(a, b, h0 + hl, s);
    a.part_o[slot * D + d] = f32_to_bf16(acc / l);  // every written chunk holds a key: l > 0
    if (d == 0) {
      a.part_ml[slot * 2 + 0] = mx;
      a.part_ml[slot * 2 + 1] = l;
    }
  }
}

// Merge the chunks of each (b, h): m* = max m_s, l* = sum 2^(m_s - m*) l_s,
// out = sum 2^(m_s - m*) l_s (o_s / l_s) / l* ("Transformer 架构完全深度解析" §十三: the running max
// and sum recurrences applied to whole chunks). Each chunk left its output normalised by its own
// sum, o_s / l_s, in bf16 (half the bytes of fp32; the merge is a convex combination of them, so
// their rounding stays within one bf16 step of the output). One wave per (b, h); a lane owns one
// 8-column group (16 bytes) c0 of the output and, when a row has fewer than 64 such groups, one
// phase of the chunks (chunks ph, ph + SPL, ...); the loads of up to 8 chunks per phase are issued
// together with that of the context length (non-temporal: each partial is read once), so a row of up
// to 8 * SPL chunks costs one round trip to memory, and the phases are summed across lanes at the end.
// The waves share nothing, so a work-group holds kMergeWaves of them (as fast as 4-wave work-groups).
constexpr int kMergeWaves = 16;
__global__ __launch_bounds__(kMergeWaves * 64) void decode_reduce_kernel(DecodeArgs a) {
  const int wid = blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= a.B * a.Nh) return;
  const int b = wid / a.Nh;
  const int h = wid % a.Nh;
  const long long slot0 = part_slot(a, b, h, 0);  // chunk s: slot0 + s * Nh
  const int nvec = a.Dv / 8;                   // 8-column groups per row (a divisor of 64)
  const int spl = 64 / nvec;                   // chunk phases
  const int c0 = lane % nvec, ph = lane / nvec;
  uint16_t* op = a.out + (long long)wid * a.Dv;
  const float* ml = a.part_ml + slot0 * 2;
  const uint16_t* po = a.part_o + slot0 * a.Dv;
  // one pass: chunks s0, s0 + spl, ... (kU of them) of this lane's phase. The slots of all nsplit
  // chunks exist, so the first pass is loaded before the context length is known (slots past the
  // sequence's last chunk hold stale data and are masked below).
  constexpr int kU = 8;
  U4 v[kU];
  float2 mls[kU];
  auto load_pass = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + u * spl;
      const bool in = s < a.nsplit;
      mls[u] = in ? *reinterpret_cast<const float2*>(ml + 2 * (long long)s * a.Nh) : make_float2(-INFINITY, 0.f);
      v[u] = in ? ldg16_nt(po + ((long long)s * a.Nh * nvec + c0) * 8) : U4{0u, 0u, 0u, 0u};
    }
  };
  const int ctx = min(max(a.ctx_lens[b], 0), a.max_ctx);
  load_pass(ph);
  const int ns = (ctx + a.chunk - 1) / a.chunk;
  if (ns == 0) {
    if (ph == 0) *reinterpret_cast<uint4*>(op + 8 * c0) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  // the reference max over the written chunks: this phase's, then across the phases
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < kU; ++u)
    if (ph + u * spl < ns) mx = fmaxf(mx, mls[u].x);
  for (int s = ph + kU * spl; s < ns; s += spl) mx = fmaxf(mx, ml[2 * (long long)s * a.Nh]);
  for (int off = nvec; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  float l = 0.f;  // sum of the weights of this lane's phase (summed over the phases below)
  auto use_pass = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + u * spl >= ns) break;
      const float wgt = mls[u].x == -INFINITY ? 0.f : fast_exp2(mls[u].x - mx) * mls[u].y;
      l += wgt;
      const uint32_t wv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(wgt, bf16lo(wv[e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(wgt, bf16hi(wv[e]), acc[2 * e + 1]);
      }
    }
  };
  use_pass(ph);
  for (int s0 = ph + kU * spl; s0 < ns; s0 += kU * spl) {
    load_pass(s0);
    use_pass(s0);
  }
  // sum the phases (lanes c0, c0 + nvec, ...) and the sums of all chunks
  for (int off = nvec; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += __shfl_xor(acc[i], off);
    l += __shfl_xor(l, off);
  }
  const float inv = 1.f / l;
  if (ph == 0)
    *reinterpret_cast<uint4*>(op + 8 * c0) =
        make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                   pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

constexpr int kDecodeNB = 2;  // LDS ring stages per wave (2: two work-groups fit a CU)

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Nh / a.Nkv;
  const int HG = G < 16 ? G : 16;
  const long long n_wg = (long long)a.B * a.Nkv * (G / HG) * a.nsplit;
  if (n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  decode_split_kernel<D, kDecodeNB><<<dim3((unsigned)n_wg), dim3(kThreads), 0, st>>>(a);
  return hipGetLastError();
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
  if (a.Dv % 8 != 0 || a.Dv > 512 || 64 % (a.Dv / 8) != 0) return hipErrorInvalidValue;
  decode_reduce_kernel<<<dim3((unsigned)((waves + kMergeWaves - 1) / kMergeWaves)), dim3(kMergeWaves * 64), 0,
                         st>>>(a);
  return hipGetLastError();
}

}  // namespace attn
