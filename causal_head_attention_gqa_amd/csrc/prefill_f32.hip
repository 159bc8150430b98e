// fp32 prefill on the vector ALUs: exact fp32 products (no reduced-precision matrix path), used
// for fp32 inputs. One lane owns one query row; K/V tiles of 32 keys are staged in LDS and read
// as broadcasts. Online softmax ("Transformer 架构完全深度解析" §十三: running max m and sum l,
// extended to the output accumulator by the same rescaling) over the tiles; tiles past the
// block's last query are never visited ("2.7 Transformer Decoder Block完整解析" §3.3).
#include "kernels.hpp"

namespace attn {

namespace {
constexpr int kRows = 64;  // query rows per block (one wave)
constexpr int kKeys = 32;  // keys per LDS tile

template <int D>
__global__ __launch_bounds__(kRows) void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                            const float* __restrict__ v, float* __restrict__ out,
                                                            const float2* __restrict__ table, int S, int Nh,
                                                            int Nkv, float c, int causal) {
  __shared__ float Ks[kKeys][D];
  __shared__ float Vs[kKeys][D];
  const int tid = threadIdx.x;
  const int p = blockIdx.x * kRows + tid;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (Nh / Nkv);

  float qr[D];
  if (p < S) {
    const float* qp = q + (((long long)b * S + p) * Nh + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] = qp[d];
    if (table) {  // half-split rotation at position p
      const float2* tb = table + (long long)p * (D / 2);
#pragma unroll
      for (int i = 0; i < D / 2; ++i) {
        const float2 cs = tb[i];
        const float a = qr[i], bb = qr[i + D / 2];
        qr[i] = a * cs.x - bb * cs.y;
        qr[i + D / 2] = a * cs.y + bb * cs.x;
      }
    }
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) qr[d] = 0.f;
  }

  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int last_row = min(S, (int)(blockIdx.x + 1) * kRows);
  const int n_keys = causal ? last_row : S;
  const long long kv_row_stride = (long long)Nkv * D;
  const float* kb = k + ((long long)b * S * Nkv + g) * D;
  const float* vb = v + ((long long)b * S * Nkv + g) * D;

  for (int j0 = 0; j0 < n_keys; j0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += kRows) {
      const int r = e / D, d = e % D;
      const int key = j0 + r;
      Ks[r][d] = key < S ? kb[key * kv_row_stride + d] : 0.f;
      Vs[r][d] = key < S ? vb[key * kv_row_stride + d] : 0.f;
    }
    __syncthreads();

    float x[kKeys];
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < kKeys; ++r) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], Ks[r][d], s);
      const int key = j0 + r;
      const bool masked = key >= S || (causal && key > p);
      x[r] = masked ? -INFINITY : s * c;
      mt = fmaxf(mt, x[r]);
    }
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float psum = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int r = 0; r < kKeys; ++r) {
      const float pr = fast_exp2(x[r] - m_use);
      psum += pr;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(pr, Vs[r][d], o[d]);
    }
    l = l * alpha + psum;
    m = m_new;
  }

  if (p < S) {
    const float inv = 1.f / l;
    float* op = out + (((long long)b * S + p) * Nh + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  }
}
}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.S + kRows - 1) / kRows), (unsigned)a.Nh, (unsigned)a.B);
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* v = static_cast<const float*>(a.v);
  float* o = static_cast<float*>(a.out);
  switch (a.D) {
    case 16:
      prefill_f32_kernel<16><<<grid, dim3(kRows), 0, st>>>(q, k, v, o, a.table, a.S, a.Nh, a.Nkv, a.scale_log2,
                                                           a.causal);
      break;
    case 32:
      prefill_f32_kernel<32><<<grid, dim3(kRows), 0, st>>>(q, k, v, o, a.table, a.S, a.Nh, a.Nkv, a.scale_log2,
                                                           a.causal);
      break;
    case 64:
      prefill_f32_kernel<64><<<grid, dim3(kRows), 0, st>>>(q, k, v, o, a.table, a.S, a.Nh, a.Nkv, a.scale_log2,
                                                           a.causal);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
