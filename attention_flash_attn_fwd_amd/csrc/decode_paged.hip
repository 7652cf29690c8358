// Paged-KV decode for gfx950: split-KV partial attention + log-sum-exp merge.
//
// One new query token per sequence attends to every cached token, whose K/V
// rows are found through a block table ("LLM推理优化技术综述" page,
// PageAttention part: the cache is cut into fixed-size blocks and a table maps
// a sequence's logical blocks to non-contiguous physical ones, like an OS
// page table; "TensorRT-LLM：大模型推理加速的工业级引擎", PagedAttention).
// Small-batch decode is bound by reading the KV cache from HBM (same page,
// decode stage), so the kernel is built around moving K/V at full bandwidth:
//  * A workgroup (4 waves) owns one (sequence, K/V head, 256-token split).
//    All Hq/Hkv query heads of the K/V head are handled together, so each
//    K/V byte is read from HBM exactly once (the GQA saving of the
//    "TensorRT对Grouped Query Attention的支持进展" page, 技术演进背景).
//  * Each wave walks 4 of the split's 16-token blocks.  A pool block of one
//    head is a contiguous 4 KiB run ([block, head, slot, dim] layout), read
//    with 16-byte loads: lane = (token row, 8-dim chunk), fully coalesced.
//  * Scores: per lane partial dot products over its 8 dims for every head,
//    summed across the chunk lanes with DPP; online softmax in base 2.
//  * P.V accumulates per lane over its own rows; rows and waves are combined
//    once per split.  The split's (O / l, log2-sum-exp) goes to the caller's
//    workspace; the merge kernel combines splits with
//    lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kBlk = 16;  // tokens per pool block
constexpr int kBlocksPerSplit = kDecodeSplitTokens / kBlk;
constexpr int kBlocksPerWave = kBlocksPerSplit / kDecWaves;
constexpr float kUnset = -1e30f;
constexpr float kLn2 = 0.69314718055994530942f;

struct DecParams {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int Hq, Hkv, num_blocks, max_blocks, n_split;
  float sl2;
};

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the CH consecutive lanes that hold one token row (CH = 8 or 16);
// every one of those lanes ends with the total.
template <int CH>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (CH == 16) x += dpp<0x128>(x);  // row_ror:8
  x += dpp<0x141>(x);                           // row_half_mirror
  x += dpp<0xB1>(x);                            // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                            // quad_perm [2,3,0,1]
  return x;
}

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecParams p) {
  constexpr int CH = D / 8;       // 16-byte chunks per token row
  constexpr int RPL = 64 / CH;    // token rows covered by one wave-wide load
  constexpr int LPB = kBlk / RPL; // loads per 16-token block
  __shared__ float sm_m[kDecWaves][G];
  __shared__ float sm_l[kDecWaves][G];
  __shared__ float sm_o[kDecWaves][G][D];
  __shared__ int sm_err;

  const int split = blockIdx.x, kvh = blockIdx.y, n = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane / CH, c = lane % CH;
  const int L = p.seq_lens[n];
  if (L <= 0 || split * kDecodeSplitTokens >= L) return;  // merge handles L <= 0
  if (tid == 0) sm_err = 0;
  __syncthreads();

  // q for the G heads of this K/V head, dims c*8..c*8+7, pre-scaled to log2 units
  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(
        p.q + ((size_t)n * p.Hq + kvh * G + h) * D + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qf[h][2 * j] = lo_bf16(w[j]) * p.sl2;
      qf[h][2 * j + 1] = hi_bf16(w[j]) * p.sl2;
    }
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kUnset;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  bool err = false;
  const int32_t* trow = p.table + (size_t)n * p.max_blocks;

  for (int jj = 0; jj < kBlocksPerWave; ++jj) {
    const int lb = split * kBlocksPerSplit + wave * kBlocksPerWave + jj;
    const int tok0 = lb * kBlk;
    if (tok0 >= L) break;
    if (lb >= p.max_blocks) { err = true; break; }
    const int phys = trow[lb];
    if (phys < 0 || phys >= p.num_blocks) { err = true; break; }
    const size_t base = (((size_t)phys * p.Hkv + kvh) * kBlk) * D + c * 8;
    u32x4 kr[LPB], vr[LPB];
#pragma unroll
    for (int rr = 0; rr < LPB; ++rr) {
      const int tok = rr * RPL + r;
      kr[rr] = *reinterpret_cast<const u32x4*>(p.k_pool + base + (size_t)tok * D);
      vr[rr] = *reinterpret_cast<const u32x4*>(p.v_pool + base + (size_t)tok * D);
    }
    float s[G][LPB];
#pragma unroll
    for (int rr = 0; rr < LPB; ++rr) {
      float kf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kf[2 * j] = lo_bf16(kr[rr][j]);
        kf[2 * j + 1] = hi_bf16(kr[rr][j]);
      }
      const bool valid = tok0 + rr * RPL + r < L;
      // slots past the sequence end hold arbitrary bits (even NaN): drop them
      // from P.V as well, since 0 * NaN would poison the accumulator
      if (!valid) vr[rr] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qf[h][e], kf[e], d);
        d = row_sum<CH>(d);
        s[h][rr] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = s[h][0];
#pragma unroll
      for (int rr = 1; rr < LPB; ++rr) bm = fmaxf(bm, s[h][rr]);
#pragma unroll
      for (int x = CH; x < 64; x <<= 1) bm = fmaxf(bm, __shfl_xor(bm, x));
      const float m_new = fmaxf(m[h], bm);
      const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
      m[h] = m_new;
      float pr[LPB];
      float ps = 0.f;
#pragma unroll
      for (int rr = 0; rr < LPB; ++rr) {
        pr[rr] = __builtin_amdgcn_exp2f(s[h][rr] - m_new);
        ps += pr[rr];
      }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int rr = 0; rr < LPB; ++rr) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[h][2 * j] = fmaf(pr[rr], lo_bf16(vr[rr][j]), acc[h][2 * j]);
          acc[h][2 * j + 1] = fmaf(pr[rr], hi_bf16(vr[rr][j]), acc[h][2 * j + 1]);
        }
      }
    }
  }

  // combine the token rows of this wave (lanes with equal chunk c)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = CH; x < 64; x <<= 1) {
      l[h] += __shfl_xor(l[h], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], x);
    }
  }
  if (err) atomicOr(&sm_err, 1);
  if (lane < CH) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][h][c * 8 + e] = acc[h][e];
      if (lane == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // combine the waves and write this split's normalised partial result
  const bool bad = sm_err != 0;
  for (int it = tid; it < G * D; it += kDecThreads) {
    const int h = it / D, d = it % D;
    float M = kUnset;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float Lsum = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float sc = __builtin_amdgcn_exp2f(sm_m[w][h] - M);
      Lsum += sc * sm_l[w][h];
      O += sc * sm_o[w][h][d];
    }
    const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
    p.ws_o[slot * D + d] = bad ? NAN : O / Lsum;
    if (d == 0) p.ws_lse[slot] = bad ? NAN : M + __log2f(Lsum);
  }
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {x, 0.f};
  return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2)) & 0xffffu);
}

// One workgroup per (query head, sequence); one thread per output dim.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecParams p) {
  const int h = blockIdx.x, n = blockIdx.y, d = threadIdx.x;
  const int L = p.seq_lens[n];
  const size_t out = ((size_t)n * p.Hq + h);
  if (L == 0) {
    p.o[out * D + d] = 0;
    if (d == 0 && p.lse) p.lse[out] = -INFINITY;
    return;
  }
  if (L < 0 || (long long)L > (long long)p.max_blocks * kBlk) {
    p.o[out * D + d] = to_bf16(NAN);
    if (d == 0 && p.lse) p.lse[out] = NAN;
    return;
  }
  const int ns = (L + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
  const float* lse_s = p.ws_lse + out * p.n_split;
  const float* o_s = p.ws_o + out * p.n_split * D;
  float M = kUnset;
  bool bad = false;
  for (int s = 0; s < ns; ++s) {
    const float v = lse_s[s];
    bad |= (v != v);
    M = fmaxf(M, v);
  }
  float W = 0.f, O = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(lse_s[s] - M);
    W += w;
    O = fmaf(w, o_s[(size_t)s * D + d], O);
  }
  O = bad ? NAN : O / W;
  p.o[out * D + d] = to_bf16(O);
  if (d == 0 && p.lse) p.lse[out] = bad ? NAN : (M + __log2f(W)) * kLn2;
}

template <int D, int G>
void launch_split(const DecParams& p, int N, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(p.n_split, p.Hkv, N), dim3(kDecThreads),
                     0, stream, p);
}

template <int D>
hipError_t launch_d(const DecParams& p, int N, int G, hipStream_t stream) {
  switch (G) {
    case 1: launch_split<D, 1>(p, N, stream); break;
    case 2: launch_split<D, 2>(p, N, stream); break;
    case 4: launch_split<D, 4>(p, N, stream); break;
    case 8: launch_split<D, 8>(p, N, stream); break;
    case 16: launch_split<D, 16>(p, N, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.Hq, N), dim3(D), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k_pool = static_cast<const uint16_t*>(a.k_pool);
  p.v_pool = static_cast<const uint16_t*>(a.v_pool);
  p.table = a.block_table;
  p.seq_lens = a.seq_lens;
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.num_blocks = a.num_blocks;
  p.max_blocks = a.max_blocks;
  p.n_split = a.n_split;
  p.sl2 = a.scale * 1.4426950408889634f;
  const int G = a.Hq / a.Hkv;
  return a.D == 64 ? launch_d<64>(p, a.N, G, stream) : launch_d<128>(p, a.N, G, stream);
}

}  // namespace attn
