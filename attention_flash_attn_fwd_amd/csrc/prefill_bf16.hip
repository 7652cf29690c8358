// bf16 exact-attention prefill for gfx950: tiled Q.K^T, online softmax and
// P.V fused in one pass, K/V tiles shared by the query heads of a GQA group.
//
// What is computed is stated on the "flash-attention与TensorRT-LLM集成" page
// (FlashAttention working principle: Q, K, V are cut into blocks that are
// processed on chip, the softmax intermediate is never written out, memory
// is linear in S) for grouped-query attention as described on the
// "TensorRT对Grouped Query Attention的支持进展" page (技术演进背景: groups of
// query heads share one K/V head; 并行化友好性: the heads of a group can cache
// their common K/V in shared memory).  The optional block skip follows the
// BLASST guide ("高效部署稀疏注意力加速方案", 架构与组件).
//
// Design (CDNA4, wave64):
//  * A workgroup is 8 waves.  It owns one K/V head and `gw` of its query
//    heads (gw = largest of 8,4,2,1 dividing Hq/Hkv) over 32*8/gw query rows;
//    every wave owns 32 query rows of one head.  Each 64-key K/V tile is read
//    from HBM/L2 once per workgroup, staged in LDS and used by all 8 waves.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read
//    from LDS, B = the wave's Q fragment held in VGPRs for the whole loop.
//    In the 32x32 accumulator each lane holds one query (column) and 16 of
//    the 32 keys, so a row maximum is an in-lane max plus one exchange with
//    lane ^ 32, and the running max/sum rescale is a per-lane scalar.
//  * O^T += V^T P^T with the same instruction: A = 32 dims x 16 keys of V^T
//    from LDS, B = P^T taken straight from the score accumulator (rounded to
//    bf16).  The reduction (k) order of an MFMA is free as long as both
//    operands agree, so V is written to LDS transposed, with the 4-key
//    chunks of each 16-key group placed in the order the accumulator hands
//    out keys; each A fragment is then one 16-byte LDS read.
//  * Softmax runs in base 2: scores are scaled by scale*log2(e) inside one
//    FMA and exponentiated with v_exp_f32.
//  * Causal: key tiles past a wave's last row are skipped per wave; only
//    diagonal tiles are masked.  Heavy query blocks are scheduled first.
#include "attn_internal.h"

#include <math.h>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int BN = 64;  // keys per K/V tile (also the block-skip tile)
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kUnset = -1e30f;  // running max before any visible key

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, S, G, gw, rows_per_wg, n_qblk, n_hgrp, sub_per_kv;
  float sl2;  // scale * log2(e)
  float thr;  // log2(lambda), block skip only
  uint8_t* skip_map;
  unsigned long long* skip_count;
  int nT;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));  // RNE
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;    // bf16 per K row in LDS (16-byte pad)
  static constexpr int VSTR = BN + 8;   // bf16 per V^T row in LDS (16-byte pad)
  static constexpr int KT = BN * KSTR;  // elements of one K tile
  static constexpr int VT = D * VSTR;   // elements of one V^T tile
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int KITEMS = BN * CH / kThreads;
  static constexpr int VITEMS = (BN / 2) * CH;  // (key pair, chunk) items
  static constexpr size_t lds_bytes = 2 * (size_t)(KT + VT) * 2;
};

template <int D, bool CAUSAL, bool SKIP>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(Params p) {
  using T = Tile<D>;
  constexpr int NKS = D / 16;  // 16-dim k-steps of Q.K^T
  constexpr int NDB = D / 32;  // 32-dim output blocks of P.V
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ int skip_flag[2][kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;

  // ---- work item: heaviest query blocks first
  const int bid = blockIdx.x;
  const int qblk = p.n_qblk - 1 - bid / p.n_hgrp;
  const int hg = bid % p.n_hgrp;
  const int sub = hg % p.sub_per_kv;
  const int bk = hg / p.sub_per_kv;
  const int kvh = bk % p.Hkv, b = bk / p.Hkv;
  const int head = kvh * p.G + sub * p.gw + (wave % p.gw);
  const int S = p.S;
  const int row0 = qblk * p.rows_per_wg;
  const int q0 = row0 + (wave / p.gw) * 32;

  const int wg_last = min(S, row0 + p.rows_per_wg) - 1;
  const int n_tiles = CAUSAL ? wg_last / BN + 1 : (S + BN - 1) / BN;
  const bool has_rows = q0 < S;
  const int wave_tiles = !has_rows ? 0 : (CAUSAL ? min(S - 1, q0 + 31) / BN + 1 : n_tiles);

  // ---- Q fragment (B operand): query q0+n, dims ks*16 + hf*8 .. +7
  const size_t qbase = ((size_t)b * p.Hq + head) * S;
  bf16x8 qf[NKS];
  {
    const int qrow = min(q0 + n, S - 1);
    const uint16_t* qp = p.q + (qbase + qrow) * D + hf * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
  }

  const size_t kvbase = ((size_t)b * p.Hkv + kvh) * (size_t)S * D;
  const uint16_t* Kg = p.k + kvbase;
  const uint16_t* Vg = p.v + kvbase;

  // ---- global -> register staging of one K/V tile
  u32x4 kreg[T::KITEMS];
  u32x4 vreg0, vreg1;
  auto load_tile = [&](int t) {
    const int c0 = t * BN;
#pragma unroll
    for (int i = 0; i < T::KITEMS; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / T::CH, c = idx % T::CH;
      const int key = c0 + r;
      kreg[i] = key < S ? *reinterpret_cast<const u32x4*>(Kg + (size_t)key * D + c * 8)
                        : u32x4{0, 0, 0, 0};
    }
    if (tid < T::VITEMS) {
      const int tp = tid / T::CH, c = tid % T::CH;
      const int key = c0 + 2 * tp;
      vreg0 = key < S ? *reinterpret_cast<const u32x4*>(Vg + (size_t)key * D + c * 8)
                      : u32x4{0, 0, 0, 0};
      vreg1 = key + 1 < S ? *reinterpret_cast<const u32x4*>(Vg + (size_t)(key + 1) * D + c * 8)
                          : u32x4{0, 0, 0, 0};
    }
  };
  // ---- register -> LDS: K row-major, V transposed and key-permuted
  auto store_tile = [&](uint16_t* kl, uint16_t* vl) {
#pragma unroll
    for (int i = 0; i < T::KITEMS; ++i) {
      const int idx = tid + i * kThreads;
      const int r = idx / T::CH, c = idx % T::CH;
      *reinterpret_cast<u32x4*>(kl + r * T::KSTR + c * 8) = kreg[i];
    }
    if (tid < T::VITEMS) {
      const int tp = tid / T::CH, c = tid % T::CH;
      // key pair (2tp, 2tp+1) lies in one 4-key chunk; within each 16-key
      // group the chunk order 0,1,2,3 is stored as 0,2,1,3
      const int key = 2 * tp;
      const int q4 = (key >> 2) & 3;
      const int posq = q4 == 1 ? 2 : (q4 == 2 ? 1 : q4);
      const int pos = (key & ~15) | (posq << 2) | (key & 3);
      const int grp = (pos >> 3) ^ (c & 7);  // 8-key group, XOR-swizzled by dim/8
      const int col = (grp << 3) | (pos & 7);
      uint16_t* dst = vl + (c * 8) * T::VSTR + col;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a = vreg0[j], bb = vreg1[j];
        const uint32_t even = (a & 0xffffu) | (bb << 16);          // dim c*8 + 2j
        const uint32_t odd = (a >> 16) | (bb & 0xffff0000u);       // dim c*8 + 2j + 1
        *reinterpret_cast<uint32_t*>(dst + (2 * j) * T::VSTR) = even;
        *reinterpret_cast<uint32_t*>(dst + (2 * j + 1) * T::VSTR) = odd;
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m = kUnset, l = 0.f;
  const float sl2 = p.sl2;

  load_tile(0);
  store_tile(smem, smem + T::KT);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const uint16_t* kl = smem + (t & 1) * (T::KT + T::VT);
    const uint16_t* vl = kl + T::KT;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const bool active = t < wave_tiles;
    const int c0 = t * BN;

    f32x16 s[2];
    float tmx = -INFINITY;
    if (active) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(kl + (kb * 32 + n) * T::KSTR + ks * 16 + hf * 8);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
        }
      }
      const bool need_mask = (c0 + BN > S) || (CAUSAL && c0 + BN - 1 > q0);
      if (need_mask) {
        const int qi = q0 + n;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = c0 + kb * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
            if (key >= S || (CAUSAL && key > qi)) s[kb][i] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      tmx = mx * sl2;
    }

    bool skip_tile = false;
    if constexpr (SKIP) {
      // BLASST test for this wave's 32 rows; the 64-row tile spans this wave
      // and the wave holding the other 32 rows (wave ^ gw).
      bool neg = true;
      if (active) {
        neg = (tmx == -INFINITY) || (m > 0.5f * kUnset && tmx - m < p.thr) || (q0 + n >= S);
      }
      const bool all_neg = __all(neg);
      if (lane == 0) skip_flag[t & 1][wave] = all_neg ? 1 : 0;
      __syncthreads();
      skip_tile = active && all_neg && skip_flag[t & 1][wave ^ p.gw];
      if (active && ((wave / p.gw) & 1) == 0 && lane == 0) {
        const int qt = q0 / BN;
        if (p.skip_map)
          p.skip_map[(((size_t)b * p.Hq + head) * p.nT + qt) * p.nT + t] = skip_tile ? 1 : 0;
        if (skip_tile && p.skip_count) atomicAdd(p.skip_count, 1ull);
      }
    }

    if (active && !skip_tile) {
      const float m_new = fmaxf(m, tmx);
      const float alpha = fast_exp2(m - m_new);
      const float nm = -m_new;
      uint32_t pk[2][8];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(s[kb][i], sl2, nm));
          const float p1 = fast_exp2(fmaf(s[kb][i + 1], sl2, nm));
          rs += p0 + p1;
          pk[kb][i >> 1] = pack_bf16(p0, p1);
        }
      l = l * alpha + rs;
      m = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 pw = {pk[kb][kk * 4 + 0], pk[kb][kk * 4 + 1], pk[kb][kk * 4 + 2],
                            pk[kb][kk * 4 + 3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
          const int lgrp = kb * 4 + kk * 2 + hf;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = db * 32 + n;
            const int col = (lgrp ^ ((d >> 3) & 7)) << 3;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vl + d * T::VSTR + col);
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
          }
        }
    }

    if (t + 1 < n_tiles) {
      uint16_t* nk = smem + ((t + 1) & 1) * (T::KT + T::VT);
      store_tile(nk, nk + T::KT);
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l (bf16, RNE), LSE = ln(sum) = (m + log2 l) ln 2
  if (!has_rows) return;
  const float lt = l + __shfl_xor(l, 32);
  const int row = q0 + n;
  if (row >= S) return;
  const float inv = 1.f / lt;
  uint16_t* orow = p.o + (qbase + row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      u32x2 w = {pack_bf16(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv),
                 pack_bf16(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + d0) = w;
    }
  if (hf == 0 && p.lse) p.lse[qbase + row] = (m + __log2f(lt)) * kLn2;
}

template <int D, bool CAUSAL, bool SKIP>
hipError_t launch_one(const Params& p, int grid, hipStream_t stream) {
  auto kern = prefill_bf16_kernel<D, CAUSAL, SKIP>;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Tile<D>::lds_bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), Tile<D>::lds_bytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
  Params p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.S = a.S;
  p.G = a.Hq / a.Hkv;
  int gw = 8;
  while (p.G % gw) gw >>= 1;
  if (a.skip && gw > 4) gw = 4;  // a 64-row skip tile must stay inside one workgroup
  p.gw = gw;
  p.rows_per_wg = 32 * kWaves / gw;
  p.n_qblk = (a.S + p.rows_per_wg - 1) / p.rows_per_wg;
  p.sub_per_kv = p.G / gw;
  p.n_hgrp = a.B * a.Hkv * p.sub_per_kv;
  p.sl2 = a.scale * 1.4426950408889634f;
  p.thr = a.skip ? (float)(log((double)a.lambda) * 1.4426950408889634) : 0.f;
  p.skip_map = a.skip_bitmap;
  p.skip_count = a.skip_count;
  p.nT = (a.S + BN - 1) / BN;
  const long long grid = (long long)p.n_qblk * p.n_hgrp;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int g = (int)grid;
  if (a.skip) {
    return a.D == 64 ? launch_one<64, true, true>(p, g, stream)
                     : launch_one<128, true, true>(p, g, stream);
  }
  if (a.causal) {
    return a.D == 64 ? launch_one<64, true, false>(p, g, stream)
                     : launch_one<128, true, false>(p, g, stream);
  }
  return a.D == 64 ? launch_one<64, false, false>(p, g, stream)
                   : launch_one<128, false, false>(p, g, stream);
}

}  // namespace attn
