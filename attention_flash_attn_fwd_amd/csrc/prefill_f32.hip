// Exact attention prefill in true float32 (no reduced-precision products).
//
// The problem is the one stated for FlashAttention on the
// "flash-attention与TensorRT-LLM集成" page (FlashAttention working principle):
// O = softmax(scale * Q K^T) V computed block by block without storing the
// S x S score matrix.  This kernel is the plain-fp32 member of the family:
// one wavefront per 64 query rows of one query head, one query row per lane,
// K/V tiles staged in LDS, a running maximum m and sum l per row (online
// softmax) and the output accumulated in registers.  It is latency-oriented
// (small shapes) rather than a throughput kernel.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (one row per lane)

template <int D, int TN>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int S, int causal,
    float scale) {
  __shared__ float ks[TN][D];
  __shared__ float vs[TN][D];
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int row = blockIdx.x * kRows + tid;
  const bool row_ok = row < S;
  const float* qrow = Q + (((size_t)b * Hq + h) * S + (row_ok ? row : S - 1)) * D;
  const float* kb = K + ((size_t)b * Hkv + g) * S * D;
  const float* vb = V + ((size_t)b * Hkv + g) * S * D;

  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qrow[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  const int last_row = min(S - 1, (int)blockIdx.x * kRows + kRows - 1);
  const int key_end = causal ? last_row + 1 : S;  // keys [0, key_end) can be visible
  for (int k0 = 0; k0 < key_end; k0 += TN) {
    __syncthreads();
    for (int e = tid; e < TN * D; e += 64) {
      const int j = e / D, d = e % D;
      const int key = k0 + j;
      ks[j][d] = key < S ? kb[(size_t)key * D + d] : 0.f;
      vs[j][d] = key < S ? vb[(size_t)key * D + d] : 0.f;
    }
    __syncthreads();
    float s[TN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int key = k0 + j;
      const bool vis = key < S && (!causal || key <= row);
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[j][d], dot);
      s[j] = vis ? dot * scale : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    if (mx == -INFINITY) continue;  // nothing visible to this row in the tile
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);  // exp(-inf) = 0 on the first visible tile
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const float p = expf(s[j] - m_new);  // 0 for masked keys
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
    m = m_new;
  }
  if (!row_ok) return;
  const float inv = 1.f / l;
  float* orow = O + (((size_t)b * Hq + h) * S + row) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  if (LSE) LSE[((size_t)b * Hq + h) * S + row] = m + logf(l);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
  dim3 grid((a.S + kRows - 1) / kRows, a.Hq, a.B);
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* v = static_cast<const float*>(a.v);
  float* o = static_cast<float*>(a.o);
  if (a.D == 64) {
    hipLaunchKernelGGL((prefill_f32_kernel<64, 16>), grid, dim3(64), 0, stream, q, k, v, o,
                       a.lse, a.Hq, a.Hkv, a.S, a.causal, a.scale);
  } else {
    hipLaunchKernelGGL((prefill_f32_kernel<128, 8>), grid, dim3(64), 0, stream, q, k, v, o,
                       a.lse, a.Hq, a.Hkv, a.S, a.causal, a.scale);
  }
  return hipGetLastError();
}

}  // namespace attn
