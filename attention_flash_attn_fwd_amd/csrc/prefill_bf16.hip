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
//    every wave owns 32 query rows of one head.  Each 64-key K/V tile is
//    copied HBM/L2 -> LDS once per workgroup (global_load_lds_dwordx4, no
//    register round trip) into a 4-stage ring and read by all 8 waves.
//    LDS rows are padded (K 16 bytes, V 64 bytes per row) so that every
//    operand read below is bank-conflict free with compile-time offsets.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims read
//    from LDS, B = the wave's Q fragment held in VGPRs for the whole loop.
//    In the 32x32 accumulator each lane holds one query (column) and 16 of
//    the 32 keys, so a row maximum is an in-lane max plus one exchange with
//    lane ^ 32 (v_permlane32_swap), and the running max/sum are per-lane.
//  * O^T += V^T P^T with the same instruction: B = P^T straight from the
//    score accumulator rounded to bf16, A = V^T fragments from the
//    transposing LDS read (ds_read_b64_tr_b16).  The reduction order of an
//    MFMA is free as long as both operands agree, so keys are taken in the
//    order the accumulator hands them out.
//  * Softmax runs in base 2 (scale * log2(e) folded into one FMA, v_exp_f32)
//    with a lazy rescale; row sums use v_dot2 on the bf16-rounded P.
//  * Ping-pong: the two waves of a SIMD alternate a pure-MFMA phase and a
//    pure-VALU (softmax) phase, half an iteration apart, so the matrix core
//    and the vector ALU work at the same time (a single wave that mixes
//    both does not overlap them on this hardware).
//  * Causal: key tiles past a wave's last row are skipped per wave; only
//    diagonal tiles are masked.  Heavy query blocks are scheduled first.
//  * A workgroup runs one to four work items (query blocks) back to back;
//    each item's last phase writes its output through LDS as whole rows and
//    copies the next item's Q and first two K/V tiles.
//  * Block skip: after the row maxima of a tile each wave votes whether its
//    rows are negligible; a 64x64 tile, whose two halves sit on the two
//    waves of one SIMD, is skipped when both vote so: it loses its P.V and
//    (in the wave that learns the decision first) its exponentials, and the
//    V tile is copied from memory only if some 64-row tile of the workgroup
//    keeps it (P.V runs one tile later to give that copy time to land).
#include "attn_internal.h"

#include <math.h>

#include <type_traits>

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

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
  // chunked prefill over a paged cache (PAGED only)
  const int32_t* cu_q;     // [N + 1] query offsets into the packed q / o / lse
  const int32_t* seq_k;    // [N] cached tokens per sequence (Sk)
  const int32_t* table;    // [N, max_blocks] block table
  int N, max_blocks, num_blocks, total_q, max_seqlen_q;
  // work items (query block x head group) and how many each workgroup runs
  int n_items, items_per_wg;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));  // RNE
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x in the lane 32 positions away (v_permlane32_swap exchanges the
// two halves of the wave); fn must be symmetric, e.g. max or add.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes at gbase + voff land at LDS byte lds_addr + 16*i.  The
// instruction is issued from asm so that the compiler does not serialise it
// against unrelated LDS reads; its completion is awaited explicitly with
// wait_vmem before the workgroup barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(gbase), "s"(m) : "memory");
}

// The same copy from a full per-lane 64-bit address (a tile gathered from
// several pool blocks has no common scalar base).
__device__ __forceinline__ void dma16_va(const void* addr, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(addr), "s"(m) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most n (wave-uniform, 0..15) vector-memory operations of
// this wave are in flight; a larger n waits for all of them.
__device__ __forceinline__ void wait_vmem_upto(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
#define ATTN_WAIT_CASE(k) \
  case k: wait_vmem<k>(); break;
    ATTN_WAIT_CASE(1) ATTN_WAIT_CASE(2) ATTN_WAIT_CASE(3) ATTN_WAIT_CASE(4) ATTN_WAIT_CASE(5)
    ATTN_WAIT_CASE(6) ATTN_WAIT_CASE(7) ATTN_WAIT_CASE(8) ATTN_WAIT_CASE(9) ATTN_WAIT_CASE(10)
    ATTN_WAIT_CASE(11) ATTN_WAIT_CASE(12) ATTN_WAIT_CASE(13) ATTN_WAIT_CASE(14) ATTN_WAIT_CASE(15)
#undef ATTN_WAIT_CASE
    default: wait_vmem<0>(); break;
  }
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS layout of one pipeline stage: a K tile then a V tile, BN rows each,
// row-major with padded rows.  K rows are D*2+16 bytes: the 16-byte K
// fragment reads of 16 consecutive rows then fall in distinct banks.  V rows
// are D*2+64 bytes: the transposing 8-byte reads of 4 rows x 64 bytes per
// half-wave fall in distinct banks.  Both paddings keep every fragment
// address a lane base plus a compile-time offset.  Tiles are filled with
// 1 KiB DMA blocks that also cover the pad slots (loaded with a dummy,
// in-bounds chunk).
template <int D>
struct Tile {
  static constexpr int CH = D / 8;            // 16-byte chunks of one row
  static constexpr int KSL = CH + 1;          // K row: slots of 16 bytes
  static constexpr int VSL = CH + 4;          // V row
  static constexpr int RB = D * 2;            // bytes of one global row
  static constexpr int RK = KSL * 16, RV = VSL * 16;
  static constexpr int KT = BN * RK;          // = KSL KiB
  static constexpr int VT = BN * RV;          // = VSL KiB
  static constexpr int STAGE = KT + VT;
  static constexpr int NST = 4;               // LDS stages: t-1 (role B), t, t+1, t+2 in flight
  static constexpr size_t lds_bytes = (size_t)NST * STAGE;
  // Block skip: K and V in rings of their own, V tile t in V stage t % 4 at
  // the start of LDS (so that every V operand read is a lane base plus an
  // immediate offset), then K tile t in K stage t % 4; the same bytes as the
  // dense layout.  A V tile is only copied once it is known to be needed
  // (see the block-skip loop).
  static constexpr uint32_t VRING = 0, KRING = NST * VT;
  static constexpr int VPW = VSL / 4;         // V copy blocks per wave of the copying group
  static_assert(VSL % 4 == 0, "a V tile splits evenly over four waves");
  static constexpr int KPW = (KSL + 3) / 4;   // K copy blocks per wave of group 1 (see issue_k)
};

#define LDS_AS __attribute__((address_space(3)))
typedef short s16x4 __attribute__((ext_vector_type(4)));

// The kernel's argument block behind a pointer the compiler cannot see
// through: the parameters are read through it once per work item, so they
// live for that item only (an item loop would otherwise hold every parameter
// in scalar registers across all items, and they would spill).
constexpr int kComputeUnits = 256;  // MI355X
// buffer resource word 3 for raw 32-bit accesses (data format 32)
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ const Params& item_params() {
  auto ptr = (const __attribute__((address_space(4))) Params*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ptr));
  return *(const Params*)ptr;
}

template <int D, bool CAUSAL, bool SKIP, bool PAGED>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(Params) {
  using T = Tile<D>;
  constexpr int NKS = D / 16;  // 16-dim k-steps of Q.K^T
  constexpr int NDB = D / 32;  // 32-dim output blocks of P.V
  constexpr int CPR = D / 8;   // 16-byte chunks per row of O
  constexpr int RPI = 64 / CPR;  // rows per wave-wide store of O
  constexpr int kOutStores = 32 / RPI + 1;  // store instructions per wave and item (O, LSE)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
  LDS_AS unsigned char* smem = (LDS_AS unsigned char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  // block skip: the votes, (tile << 1) | negligible, for even and odd tiles,
  // then a landing area for the lanes of a vote write that carry no vote
  __shared__ __attribute__((aligned(16))) int vote_lds[3 * kWaves + 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  // ---- work items.  Workgroup g of G runs items g, 2G-1-g, 2G+g, 4G-1-g,
  // ... (items_per_wg of them, those below n_items).  Items are numbered
  // heaviest query block first, so each pair holds a heavy and a light
  // block and the workgroups of a causal launch get equal tile counts.  An
  // item's last phase issues the next item's Q and first two tiles, and its
  // output stores drain while the next item starts.  The tile stages run on
  // as one ring across items (ring = stage of the item's tile 0).
  const int nwg = gridDim.x;
  auto item_bid = [&](int it) {
    return (it >> 1) * 2 * nwg + ((it & 1) ? 2 * nwg - 1 - (int)blockIdx.x : (int)blockIdx.x);
  };
  const int grp = wave >> 2;  // wave group of the ping-pong (see the tile loop)
  bf16x8 qf[NKS];           // Q fragments (B operand): query q0+n, dims ks*16 + hf*8 .. +7
  bool prefetched = false;  // Q and tiles 0, 1 of this item were issued by the previous one
  int ring = 0;
  for (int it = 0;; ++it) {
    const Params& p = item_params();
    const int bid = item_bid(it);
    // ---- work item: heaviest query blocks first (paged: across sequences)
    const int hg = bid % p.n_hgrp;
    const int seq = PAGED ? (bid / p.n_hgrp) % p.N : 0;
    const int qblk = p.n_qblk - 1 - (PAGED ? bid / p.n_hgrp / p.N : bid / p.n_hgrp);
    const int sub = hg % p.sub_per_kv;
    const int bk = hg / p.sub_per_kv;
    const int kvh = bk % p.Hkv, b = bk / p.Hkv;
    // Waves w and w+4 share a SIMD and run the tile loop half an iteration
    // apart (see below), so they get adjacent 32-row slots: equal causal tile
    // counts keep both busy to the end.  With block skip they hold the two
    // halves of one 64-row skip tile (same head, rows r .. r+31 and r+32 ..
    // r+63), which the decisions rely on (see the block-skip loop); for
    // gw == 1 that is the same mapping.
    const int kq = wave & 3;
    const int slot = SKIP ? (kq % p.gw) + p.gw * (2 * (kq / p.gw) + (wave >> 2)) : (kq << 1) | (wave >> 2);
    const int head = kvh * p.G + sub * p.gw + (slot % p.gw);
    const int row0 = qblk * p.rows_per_wg;
    const int q0 = row0 + (slot / p.gw) * 32;
    // Sq query rows at key positions off .. off+Sq-1 of Sk keys (dense: all S)
    int Sq = p.S, Sk = p.S, off = 0, qstart = 0;
    if constexpr (PAGED) {
      // The sequence's device-side description is checked before anything
      // is read through it: query offsets inside [0, total_q] and in order,
      // at most max_seqlen_q queries (the grid's reach), Sq <= Sk <= the
      // table row, and every table entry its keys use inside the pool.  A
      // sequence that breaks any of these gets NaN in O and LSE for its
      // rows, clamped to [0, total_q), and nothing else is read or written.
      const int lo = p.cu_q[seq], hi = p.cu_q[seq + 1];
      Sk = p.seq_k[seq];
      bool bad = lo < 0 || hi > p.total_q || hi < lo || hi - lo > p.max_seqlen_q || Sk < 0 ||
                 Sk > p.max_blocks * 16 || hi - lo > Sk;
      if (!bad) {
        const int32_t* trow = p.table + (size_t)seq * p.max_blocks;
        bool bad_entry = false;
        for (int x = lane; x < (Sk + 15) >> 4; x += 64) {
          const int e = trow[x];
          bad_entry = bad_entry || e < 0 || e >= p.num_blocks;
        }
        bad = __any(bad_entry);
      }
      if (bad) {
        // every workgroup of the sequence covers its query block and the
        // blocks n_qblk, 2 n_qblk, ... after it, so all rows get NaN
        const int r_lo = max(lo, 0), r_hi = min(hi, p.total_q);
        for (int row = r_lo + q0 + n; row < r_hi; row += p.n_qblk * p.rows_per_wg) {
          uint16_t* orow = p.o + ((size_t)row * p.Hq + head) * D;
          for (int d = hf * 4; d < D; d += 8)
            *reinterpret_cast<u32x2*>(orow + d) = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
          if (hf == 0 && p.lse) p.lse[(size_t)row * p.Hq + head] = NAN;
        }
        return;
      }
      qstart = lo;
      Sq = hi - lo;
      off = Sk - Sq;
      if (row0 >= Sq) return;  // whole workgroup past this chunk
    }
    const int S = Sk;  // key count

    const int wg_last = min(Sq, row0 + p.rows_per_wg) - 1;
    const int n_tiles = CAUSAL ? (off + wg_last) / BN + 1 : (S + BN - 1) / BN;
    const bool has_rows = q0 < Sq;
    const int wave_tiles = !has_rows ? 0 : (CAUSAL ? (off + min(Sq - 1, q0 + 31)) / BN + 1 : n_tiles);
    // whether the workgroup has a next item (dense prefill only)
    auto has_next = [&]() {
      return !PAGED && !SKIP && it + 1 < p.items_per_wg && item_bid(it + 1) < p.n_items;
    };

    const size_t kvbase = ((size_t)b * p.Hkv + kvh) * (size_t)S * D;
    const uint16_t* Kg = p.k + kvbase;
    const uint16_t* Vg = p.v + kvbase;
    // LDS byte offsets of K tile t and V tile t (dense: one ring of K+V
    // stages continuing across items; block skip: separate K and V rings)
    auto k_stage = [&](int t) -> uint32_t {
      return SKIP ? T::KRING + (uint32_t)(t & 3) * T::KT : (uint32_t)((t + ring) % T::NST) * T::STAGE;
    };
    auto v_stage = [&](int t) -> uint32_t {
      return SKIP ? T::VRING + (uint32_t)(t & 3) * T::VT
                  : (uint32_t)((t + ring) % T::NST) * T::STAGE + T::KT;
    };

    // ---- asynchronous global -> LDS copy of tile t into stage t % NST.
    // One wave-wide load fills 1 KiB of LDS (16 bytes per lane, in lane
    // order); the lane fetches the global chunk that the padded layout puts
    // there.  The NBLK blocks of a stage (K blocks 0 .. KSL-1, then V blocks)
    // are numbered jointly and dealt round robin, block w + 8j to wave w, so
    // every wave issues DMA_LO or DMA_HI of them; since the K tile is exactly
    // KSL KiB, block i always lands at byte i KiB of the stage.  Slot g of a
    // block is row g / SL, chunk g % SL (a pad slot re-reads chunk 0 of its
    // row).  The per-lane source offsets are fixed for every tile: the tile's
    // first key enters through the scalar base address.  Keys past the end
    // are clamped to the last key and masked later.
    constexpr int NBLK = T::KSL + T::VSL;
    constexpr int DMA_HI = (NBLK + kWaves - 1) / kWaves, DMA_LO = NBLK / kWaves;
    const bool dma_hi = wave < NBLK % kWaves;
    uint32_t doff[DMA_HI];  // row * RB + chunk offset
    int drow[DMA_HI];
#pragma unroll
    for (int j = 0; j < DMA_HI; ++j) {
      const int i = wave + j * kWaves;
      const bool is_k = i < T::KSL;
      const int sl = is_k ? T::KSL : T::VSL;
      const int g = (is_k ? i : i - T::KSL) * 64 + lane, c = g % sl;
      drow[j] = g / sl;
      doff[j] = (uint32_t)drow[j] * T::RB + (c < T::CH ? c : 0) * 16;
    }
    // Paged, whole tiles: the lane's row r of slot j lies in pool block r / 16
    // of the tile's four, at the same offset in every tile, so pool + that
    // offset is fixed per item and a copy adds the block's base (entry x
    // block bytes).  A slot's rows touch at most two adjacent pool blocks.
    const unsigned char* pvrow[DMA_HI];
    if constexpr (PAGED) {
#pragma unroll
      for (int j = 0; j < DMA_HI; ++j) {
        const int i = wave + j * kWaves;
        const int r = drow[j];
        pvrow[j] = reinterpret_cast<const unsigned char*>(i < T::KSL ? p.k : p.v) +
                   (((size_t)kvh << 4) + (r & 15)) * T::RB + (doff[j] - (uint32_t)r * T::RB);
      }
    }
    // Dense tile t of the item whose K and V start at kg and vg, into stage
    // (t + rg) % NST.
    auto issue_dense = [&](const uint16_t* kg, const uint16_t* vg, int t, int rg) {
      const uint32_t st = smem_base + ((t + rg) % T::NST) * T::STAGE;
      const int key0 = t * BN;
      const uint16_t* kb_ = kg + (size_t)key0 * D;
      const uint16_t* vb_ = vg + (size_t)key0 * D;
      if (key0 + BN <= S) {
#pragma unroll
        for (int j = 0; j < DMA_HI; ++j) {
          const int i = wave + j * kWaves;
          if (j == DMA_LO && !dma_hi) break;
          dma16(i < T::KSL ? kb_ : vb_, doff[j], st + i * 1024);
        }
      } else {
        const int lim = S - 1 - key0;  // clamp keys past the end to the last key
#pragma unroll
        for (int j = 0; j < DMA_HI; ++j) {
          const int i = wave + j * kWaves;
          if (j == DMA_LO && !dma_hi) break;
          const uint32_t o = doff[j] - (uint32_t)(drow[j] - min(drow[j], lim)) * T::RB;
          dma16(i < T::KSL ? kb_ : vb_, o, st + i * 1024);
        }
      }
    };
    auto issue = [&](int t) {
      if constexpr (PAGED) {
        const uint32_t st = smem_base + ((t + ring) % T::NST) * T::STAGE;
        const int key0 = t * BN;
        // the tile's 4 pool blocks (table entries clamped into the pool)
        // The table is read through the constant address space: the entries
        // are uniform and read-only, so they come by scalar loads, which the
        // copy waits (vector-memory counts) do not see.  A vector load here
        // would make the compiler wait for it with vmcnt(0) before the use,
        // draining every tile copy in flight.  Entries past the sequence's
        // last block are never selected (keys past the end are clamped to
        // the last key), so their index is clamped instead of tested.
        const __attribute__((address_space(4))) int32_t* trow =
            (const __attribute__((address_space(4))) int32_t*)(p.table + (size_t)seq * p.max_blocks);
        const int nbs = (S + 15) >> 4;
        int e[4];
        if (t * 4 + 3 < nbs) {  // four adjacent entries: one scalar load
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = trow[t * 4 + x];
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = trow[min(t * 4 + x, nbs - 1)];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = min(max(e[x], 0), p.num_blocks - 1);
        if (key0 + BN <= S) {
          const uint32_t bs = (uint32_t)p.Hkv * 16 * T::RB;  // bytes of one pool block
#pragma unroll
          for (int j = 0; j < DMA_HI; ++j) {
            const int i = wave + j * kWaves;
            if (j == DMA_LO && !dma_hi) break;
            // the slot's first pool block (uniform) and, per lane, it or the next
            const int x0 = __builtin_amdgcn_readfirstlane(drow[j]) >> 4;
            const int ea = x0 == 0 ? e[0] : x0 == 1 ? e[1] : x0 == 2 ? e[2] : e[3];
            const int eb = x0 == 0 ? e[1] : x0 == 1 ? e[2] : e[3];
            const uint32_t ph = (uint32_t)((drow[j] >> 4) == x0 ? ea : eb);
            dma16_va(pvrow[j] + (size_t)ph * bs, st + i * 1024);
          }
          return;
        }
        const unsigned char* kpool = reinterpret_cast<const unsigned char*>(p.k);
        const unsigned char* vpool = reinterpret_cast<const unsigned char*>(p.v);
#pragma unroll
        for (int j = 0; j < DMA_HI; ++j) {
          const int i = wave + j * kWaves;
          if (j == DMA_LO && !dma_hi) break;
          const int r = drow[j];
          const int key = key0 + min(r, S - 1 - key0);
          const int bl = (key >> 4) - t * 4;
          const int ph = bl == 0 ? e[0] : bl == 1 ? e[1] : bl == 2 ? e[2] : e[3];
          const uint32_t choff = doff[j] - (uint32_t)r * T::RB;
          const unsigned char* pool = i < T::KSL ? kpool : vpool;
          dma16_va(pool + ((((size_t)ph * p.Hkv + kvh) << 4) + (key & 15)) * T::RB + choff,
                   st + i * 1024);
        }
      } else {
        issue_dense(Kg, Vg, t, ring);
      }
    };
    // Block skip: K and V tiles are copied separately, each by one wave
    // group and dealt round robin to its four waves: group 0 copies every K
    // tile (tile j+2 in its VALU phase j), group 1 the V tiles that the
    // decisions keep (see the block-skip loop).  Every group-0 wave issues
    // KPW blocks of a K tile: a wave with one block fewer copies its last
    // block twice (the same bytes to the same place), so that its count of
    // copies in flight, and with it the wait at the end of a phase, is fixed.
    // Slot g of a block is row g / SL, chunk g % SL, as above; keys past the
    // end are clamped to the last key.
    const int kb_last = kq + 4 * (T::KPW - 1) < T::KSL ? kq + 4 * (T::KPW - 1) : kq + 4 * (T::KPW - 2);
    auto kblk = [&](int j) { return j == T::KPW - 1 ? kb_last : kq + 4 * j; };
    auto slot_off = [&](int g, int sl) -> uint32_t {
      const int r = g / sl, c = g % sl;
      return (uint32_t)r * T::RB + (c < T::CH ? c : 0) * 16;
    };
    // a wave's own copy offsets: K blocks in group 0, V blocks in group 1
    constexpr int NOFF = T::KPW > T::VPW ? T::KPW : T::VPW;
    uint32_t coff[SKIP ? NOFF : 1];
    if constexpr (SKIP) {
#pragma unroll
      for (int j = 0; j < NOFF; ++j) {
        coff[j] = grp == 0 ? slot_off(kblk(j < T::KPW ? j : 0) * 64 + lane, T::KSL)
                           : slot_off((kq + 4 * j) * 64 + lane, T::VSL);
        asm volatile("" : "+v"(coff[j]));  // kept whole (its parts cost registers)
      }
    }
    // offset o of this lane's slot of block i of a block array with sl
    // slots per row, with rows past lim clamped to row lim
    auto clamp_off = [&](uint32_t o, int i, int sl, int lim) -> uint32_t {
      // (the lane index passes through an empty asm so that the row is
      // formed here, in the rare ragged copy, instead of being hoisted and
      // kept for the whole item, which cost registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r = (i * 64 + ln) / sl;
      return o - (uint32_t)(r - min(r, lim)) * T::RB;
    };
    // (whole: the caller knows that tile t has all BN keys)
    auto issue_k = [&](int t, bool whole) {  // a group-0 wave's KPW blocks of K tile t
      const uint32_t st = smem_base + k_stage(t);
      const int key0 = t * BN;
      const uint16_t* src = Kg + (size_t)key0 * D;
      if (whole || key0 + BN <= S) {
#pragma unroll
        for (int j = 0; j < T::KPW; ++j) dma16(src, coff[j], st + kblk(j) * 1024);
      } else {
#pragma unroll
        for (int j = 0; j < T::KPW; ++j) {
          const int i = kblk(j);
          dma16(src, clamp_off(coff[j], i, T::KSL, S - 1 - key0), st + i * 1024);
        }
      }
    };
    auto issue_v = [&](int t, bool whole) {  // a group-1 wave's VPW blocks of V tile t
      const uint32_t st = smem_base + v_stage(t);
      const int key0 = t * BN;
      const uint16_t* src = Vg + (size_t)key0 * D;
      if (whole || key0 + BN <= S) {
#pragma unroll
        for (int j = 0; j < T::VPW; ++j) dma16(src, coff[j], st + ((wave & 3) + 4 * j) * 1024);
      } else {
#pragma unroll
        for (int j = 0; j < T::VPW; ++j) {
          const int i = (wave & 3) + 4 * j;
          dma16(src, clamp_off(coff[j], i, T::VSL, S - 1 - key0), st + i * 1024);
        }
      }
    };
    auto issue_v_all = [&](int t) {  // every block of V tile t, from this wave
      const uint32_t st = smem_base + v_stage(t);
      const int key0 = t * BN;
      const uint16_t* src = Vg + (size_t)key0 * D;
      for (int i = 0; i < T::VSL; ++i) {
        int g = i * 64 + lane;
        asm volatile("" : "+v"(g));
        dma16(src, clamp_off(slot_off(g, T::VSL), i, T::VSL, S - 1 - key0), st + i * 1024);
      }
    };

    // wait until only the DMA blocks of the newest tile are in flight
    auto wait_all_but_newest = [&]() {
      if (DMA_HI == DMA_LO || !dma_hi) wait_vmem<DMA_LO>(); else wait_vmem<DMA_HI>();
    };

    // ---- Q fragment (B operand): query q0+n, dims ks*16 + hf*8 .. +7
    const size_t qbase = ((size_t)b * p.Hq + head) * Sq;
    // element offset of query row r (dense [B,Hq,S,D]; paged packed [total_q,Hq,D])
    auto qrow_off = [&](int r) -> size_t {
      return PAGED ? ((size_t)(qstart + r) * p.Hq + head) * D : (qbase + r) * D;
    };
    if (!prefetched) {
      const int qrow = min(q0 + n, Sq - 1);
      const uint16_t* qp = p.q + qrow_off(qrow) + hf * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16);
      // The first two tile copies go out together with the Q loads; then one
      // wait the compiler can see (vmcnt(0)) completes all of them, so it
      // places no vector-memory waits of its own inside the loop, where they
      // would also drain the tile prefetches.
      if constexpr (SKIP) {
        if (grp == 0) {
          issue_k(0, false);
          if (n_tiles > 1) issue_k(1, false);
        }
      } else {
        issue(0);
        if (n_tiles > 1) issue(1);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
      // Q (in this wave's output slice of the previous item) and tiles 0 and
      // 1 were copied by the previous item, ahead of its output stores, which
      // may still be in flight
      wait_vmem<kOutStores>();
      const LDS_AS unsigned char* qs =
          smem + ((ring + 2 + grp) % T::NST) * T::STAGE + (wave & 3) * (32 * D * 2);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = *reinterpret_cast<const LDS_AS bf16x8*>(qs + (n * CPR + ((2 * ks + hf) ^ (n % CPR))) * 16);
      // read before tile 2 or 3 of this item can land in the slice
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    // per-lane LDS offsets of the MFMA operand reads (see Tile)
    const int k_base = n * T::RK + hf * 16;                 // + kb*32*RK + ks*32
    const int vg = lane >> 4, vs = lane & 15;
    const int v_base = ((vg >> 1) * 4 + (vs >> 2)) * T::RV + ((vg & 1) * 16 + 4 * (vs & 3)) * 2;

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    float m_used = kUnset;   // reference max of the exponentials (log2 units)
    float m_true = kUnset;   // running max over the tiles before the current one
    float l = 0.f;
    unsigned skipped = 0;
    const float sl2 = p.sl2;
    const float thr = p.thr;  // block skip: log2(lambda)
    const int first_masked = CAUSAL ? min((off + q0) / BN, S / BN) : S / BN;

    // S^T of key tile t (raw scores) = K Q^T: two independent 32-key
    // accumulator chains, operand reads running ahead of the MFMAs
    auto qk = [&](int t, f32x16* sc) {
      const LDS_AS unsigned char* kp = smem + k_stage(t) + k_base;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[0][i] = sc[1][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a0 = *reinterpret_cast<const LDS_AS bf16x8*>(kp + ks * 32);
        const bf16x8 a1 = *reinterpret_cast<const LDS_AS bf16x8*>(kp + 32 * T::RK + ks * 32);
        sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], sc[0], 0, 0, 0);
        sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], sc[1], 0, 0, 0);
      }
      // 4 operand reads ahead, then alternate MFMA / read
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NKS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // Q.K^T of keys kb*32 .. kb*32+31 of tile t alone, into acc (block
    // skip: the recompute of a tile, one 32-key half at a time)
    auto qk_half = [&](int t, int kb, f32x16& acc_) {
      const LDS_AS unsigned char* kp = smem + k_stage(t) + k_base + kb * 32 * T::RK;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_[i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const LDS_AS bf16x8*>(kp + ks * 32);
        acc_ = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc_, 0, 0, 0);
      }
    };
    // mask (diagonal and ragged tiles only) and scaled row max of a score tile
    auto mask_tile = [&](int t, f32x16* sc) {
      if (t >= first_masked) {
        const int c0 = t * BN, qi = q0 + n;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = c0 + kb * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
            if (key >= S || (CAUSAL && key > off + qi)) sc[kb][i] = -INFINITY;
          }
      }
    };
    auto tile_max = [&](const f32x16* sc) -> float {
      float m0 = fmaxf(sc[0][0], sc[1][0]), m1 = fmaxf(sc[0][1], sc[1][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        m0 = fmaxf(fmaxf(m0, sc[0][i]), sc[1][i]);
        m1 = fmaxf(fmaxf(m1, sc[0][i + 1]), sc[1][i + 1]);
      }
      return half_swap_max(fmaxf(m0, m1)) * sl2;
    };
    auto row_max = [&](int t, f32x16* sc) -> float {
      mask_tile(t, sc);
      return tile_max(sc);
    };
    // softmax of a score tile into bf16 P (packed for the P.V MFMA).  The
    // exponent reference moves (with a rescale of O and l) only when the row
    // max grew by more than 8, a factor 256; the result is exact after 1/l.
    // With block skip, P.V runs a tile later than the softmax (below), so
    // when the reference moves, the P of the previous tile is still on its
    // way into acc: the rescale of acc is then held (alpha_pend) and applied
    // at the start of the next VALU phase, once that P.V has been added.
    float alpha_pend = 1.f;
    bool pend = false;
    auto apply_pending = [&]() {
      if (pend) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha_pend;
        pend = false;
      }
    };
    // the lazy rescale for a tile whose scaled row max is tmx
    auto rescale = [&](float tmx) {
      if (__any(tmx > m_used + 8.f)) {
        const float m_new = fmaxf(m_used, tmx);
        const float alpha = fast_exp2(m_used - m_new);
        l *= alpha;
        if constexpr (SKIP) {
          alpha_pend = alpha;
          pend = true;
        } else {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
        m_used = m_new;
      }
    };
    // P = exp2(scores * sl2 + nm) rounded to bf16 (nm = -m_used); returns
    // the row sum of the bf16-rounded P (the values P.V uses), two per dot2
    auto exps = [&](f32x16* sc, uint32_t (*pk)[8], float nm) -> float {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2)
          pk[kb][i >> 1] = pack_bf16(fast_exp2(fmaf(sc[kb][i], sl2, nm)),
                                     fast_exp2(fmaf(sc[kb][i + 1], sl2, nm)));
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[0][j]), kOnes2, rs0, false);
        rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[1][j]), kOnes2, rs1, false);
      }
      return rs0 + rs1;
    };
    auto softmax = [&](f32x16* sc, float tmx, uint32_t (*pk)[8]) {
      rescale(tmx);
      l += exps(sc, pk, -m_used);
    };
    // O^T += V^T P^T for key tile t; V^T fragments come from the transposing
    // LDS read, running ahead of the MFMAs
    auto pv = [&](int t, uint32_t (*pk)[8]) {
      const LDS_AS unsigned char* vl = smem + v_stage(t) + v_base;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 pw = {pk[kb][kk * 4 + 0], pk[kb][kk * 4 + 1], pk[kb][kk * 4 + 2],
                            pk[kb][kk * 4 + 3]};
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const LDS_AS unsigned char* va = vl + (kb * 32 + kk * 16) * T::RV + db * 64;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)va);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(va + 8 * T::RV));
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
          }
        }
      // three MFMAs' operands ahead, then alternate one MFMA / two reads
      constexpr int NM = 4 * NDB;
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < NM - 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    };
    // Block skip: each wave votes on key tile t (are all 32 of its rows
    // negligible?) in its VALU phase t, into an LDS slot of its own (one set
    // for even tiles, one for odd ones); a 64-row tile is skipped when both
    // of its waves, w and w+4, vote so.  The votes need no waiting: group 1
    // reads group 0's votes on t in its own VALU phase t, which follows
    // group 0's behind a barrier, and group 0 reads its partner's vote on t
    // in its VALU phase t+1, behind the next barrier.  A slot is rewritten
    // two tiles later, after both readers are done.  Lane 0 writes the vote;
    // the other lanes of the same write land in a scratch area, which spares
    // switching lanes off and on.
    LDS_AS int* const vote_w =
        (LDS_AS int*)&vote_lds[0] + (lane == 0 ? wave : 2 * kWaves + lane - 1);
    // lanes whose query row is past the end vote "negligible" on every tile
    const uint64_t rows_out = __ballot(q0 + n >= S);
    // 1 if every row of this wave is negligible on tile t (so when not live)
    auto vote_publish = [&](int t, float tmx_t, bool live) -> int {
      int all_neg = 1;
      if (live) {
        const bool neg = (tmx_t == -INFINITY) | ((m_true > 0.5f * kUnset) & (tmx_t - m_true < thr));
        all_neg = (__ballot(neg) | rows_out) == ~0ull ? 1 : 0;
      }
      __hip_atomic_store(vote_w + (t & 1) * kWaves, all_neg, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
      return all_neg;
    };
    // group 1: lanes 0-3 read group 0's votes on tile t (lane w = wave w)
    const LDS_AS int* const vote_r0 = (const LDS_AS int*)&vote_lds[0] + (lane & 3);
    auto read_votes0 = [&](int t) -> int { return *(volatile const LDS_AS int*)(vote_r0 + (t & 1) * kWaves); };
    // group 0: its partner's (wave + 4) vote on tile t, in every lane
    const LDS_AS int* const vote_rp = (const LDS_AS int*)&vote_lds[0] + wave + 4;
    auto read_partner = [&](int t) -> int { return *(volatile const LDS_AS int*)(vote_rp + (t & 1) * kWaves); };
    // Group 1 records the decisions on its 64-row tile's live tiles (it
    // learns each one in the tile's phase): bit t % 64 of rec (a
    // wave-uniform value) for tile t, written to the bitmap a byte per lane
    // and tile when a group of 64 tiles is complete, and at the end (a store
    // per tile cost 8%).  The buffer resource ends at the tile row's last
    // live tile (rec_tiles), so the range check drops the rest.
    const int records = SKIP && grp == 1 && q0 - 32 < Sq ? 1 : 0;
    const int rec_tiles = records ? (off + min(Sq - 1, q0 + 31)) / BN + 1 : 0;
    uint64_t rec = 0;
    auto record = [&](int t, int sk) { rec |= (uint64_t)(sk & records) << (t & 63); };
    auto flush_skips = [&](int t0) {
      uint8_t* row = p.skip_map == nullptr
                         ? nullptr
                         : p.skip_map + (((size_t)b * p.Hq + head) * p.nT + q0 / BN) * p.nT;
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row ? rec_tiles : 0, kBufferFlags);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)((rec >> lane) & 1), rs, t0 + lane, 0, 0);
      skipped += (unsigned)__builtin_popcountll(rec);
      rec = 0;
    };
    // a full group of 64 decisions is written in the phase of its last tile
    auto flush_due = [&](int t) { return records && t < rec_tiles && (t & 63) == 63; };

    // The last phase pair of the item: P.V of its last tile, then a VALU
    // phase with no tile work left, which takes the epilogue and, when the
    // workgroup has a next item, that item's Q and first two tiles.
    //  * O = acc / l (bf16, RNE) goes through a private LDS slice and leaves
    //    as whole rows, 16 bytes per lane (the accumulator holds 8-byte pieces
    //    of a row per lane).  Group 0's slices sit in the stage of tile n-2,
    //    group 1's in that of tile n-1: nobody reads them any more when the
    //    group gets here (group 1 reads tile n-1 during group 0's last VALU
    //    phase, which is why group 0 does not use it).  Chunk c of row r sits
    //    at chunk c ^ (r % CPR) of the slice row, spreading a column of chunks
    //    over the banks.  LSE = ln(sum) = (m + log2 l) ln 2.
    //  * The stores go through buffer resources that cover exactly this
    //    wave's valid rows (the range check drops the rest), so every wave
    //    issues kOutStores of them, as its last vector-memory operations of
    //    the item; the next item's first wait leaves them in flight.
    //  * Once the slice has been read back, the next item's Q rows land in it
    //    by LDS copy (same swizzle), and its tiles 0 and 1 go to the two
    //    stages after this item's last one (they held tiles n-4 and n-3).
    auto finish = [&](bool do_pv, uint32_t (*pk)[8]) {
      if (do_pv) pv(n_tiles - 1, pk);
      block_barrier();
      if constexpr (SKIP) {
        if (records && (rec_tiles & 63) != 0) flush_skips((rec_tiles - 1) & ~63);  // the last group
        if (lane == 0 && skipped && p.skip_count)
          atomicAdd(p.skip_count, (unsigned long long)skipped);
      }
      const float lt = half_swap_add(l);
      const float inv = 1.f / lt;
      static_assert(4 * 32 * D * 2 <= T::STAGE, "four output slices must fit in a stage");
      static_assert(2 * 4 * 32 * D * 2 <= T::NST * T::KT, "eight output slices must fit in the K ring");
      // block skip: group g's slices in the K ring, free once the last Q.K^T is done
      const uint32_t slice = (SKIP ? T::KRING + (uint32_t)grp * (4 * 32 * D * 2)
                                   : ((ring + n_tiles + 2 + grp) % T::NST) * T::STAGE) +
                             (wave & 3) * (32 * D * 2);
      LDS_AS unsigned char* ost = smem + slice;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x2 w = {pack_bf16(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv),
                           pack_bf16(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv)};
          const int c = (db * 4 + g4) ^ (n % CPR);
          *reinterpret_cast<LDS_AS u32x2*>(ost + n * (D * 2) + c * 16 + hf * 8) = w;
        }
      u32x4 ow[32 / RPI];
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / CPR, c = lane % CPR;
        ow[i] = *reinterpret_cast<const LDS_AS u32x4*>(ost + r * (D * 2) + (c ^ (r % CPR)) * 16);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // slice read back before it is refilled
      if (has_next()) {
        const int next_bid = item_bid(it + 1);
        const int nhg = next_bid % p.n_hgrp;
        const int nqblk = p.n_qblk - 1 - next_bid / p.n_hgrp;
        const int nbk = nhg / p.sub_per_kv;
        const int nkvh = nbk % p.Hkv, nb = nbk / p.Hkv;
        const int nhead = nkvh * p.G + (nhg % p.sub_per_kv) * p.gw + (slot % p.gw);
        const int nrow0 = nqblk * p.rows_per_wg;
        const int nq0 = nrow0 + (slot / p.gw) * 32;
        const int nn_tiles = CAUSAL ? (min(S, nrow0 + p.rows_per_wg) - 1) / BN + 1 : (S + BN - 1) / BN;
        const uint16_t* nqh = p.q + ((size_t)nb * p.Hq + nhead) * (size_t)S * D;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int sl = i * 64 + lane, r = sl / CPR, c = (sl % CPR) ^ (r % CPR);
          dma16(nqh, (uint32_t)(min(nq0 + r, S - 1) * (D * 2) + c * 16), smem_base + slice + i * 1024);
        }
        const size_t nkv = ((size_t)nb * p.Hkv + nkvh) * (size_t)S * D;
        issue_dense(p.k + nkv, p.v + nkv, 0, ring + n_tiles);
        if (nn_tiles > 1) issue_dense(p.k + nkv, p.v + nkv, 1, ring + n_tiles);
      }
      const int nvalid = has_rows ? min(32, Sq - q0) : 0;
      const int ostride = (PAGED ? p.Hq : 1) * D * 2;  // bytes from one row of O to the next
      const auto orsrc = __builtin_amdgcn_make_buffer_rsrc(
          p.o + (has_rows ? qrow_off(q0) : 0), (short)0,
          nvalid > 0 ? (nvalid - 1) * ostride + D * 2 : 0, kBufferFlags);
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(ow[i], orsrc, (i * RPI + lane / CPR) * ostride + (lane % CPR) * 16, 0, 0);
      const int lstride = (PAGED ? p.Hq : 1) * 4;
      float* lrow0 = p.lse == nullptr || !has_rows
                         ? p.lse
                         : p.lse + (PAGED ? (size_t)(qstart + q0) * p.Hq + head : qbase + q0);
      const auto lrsrc = __builtin_amdgcn_make_buffer_rsrc(
          lrow0, (short)0, (p.lse != nullptr && nvalid > 0) ? (nvalid - 1) * lstride + 4 : 0, kBufferFlags);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((m_used + __log2f(lt)) * kLn2), lrsrc,
                                            n * lstride, 0, 0);  // both halves hold the same value
      block_barrier();
      if (grp == 0) block_barrier();
    };

    f32x16 sc[2];
    if constexpr (!SKIP) {
      // Ping-pong.  Each wave alternates an MFMA phase (P.V of tile j-1, then
      // Q.K^T of tile j) and a VALU phase (mask, row max and softmax of tile
      // j), separated by workgroup barriers.  The second wave of each SIMD
      // (waves 4-7, group 1) runs one barrier behind the first, so at every
      // moment one wave of the pair feeds the matrix core while the other's
      // exponentials run on the vector ALU; a wave that mixed both kinds of
      // work in one stream would not overlap them.  Both groups run the same
      // code, so the scores and P never need registers at the same time.
      //
      // DMA: group 0 issues its share of tile j+2 in its VALU phase j, group
      // 1 its share of tile j+3 (and of tile 2 in its extra first slot); the
      // issue stalls the issuing wave, and an MFMA-phase wave would hold the
      // matrix core idle meanwhile.  The stage a share overwrites was last
      // read before the preceding barrier.  At the end of its VALU phase j
      // every wave waits until only the share it has just issued is in
      // flight: group 0's share of tile j+1 is then complete at the barrier
      // after which the first Q.K^T of tile j+1 starts, group 1's share of
      // tile j+2 a half iteration before the corresponding barrier.
      //
      // The iterations in which every step is present (no causal mask, no
      // pipeline start or end) run a copy of the body without the tests.
      uint32_t pk[2][8];
      block_barrier();
      if (grp == 1) {
        if (2 < n_tiles) issue(2);
        block_barrier();
      }
      auto general = [&](int j) {
        if (j >= 1 && j - 1 < wave_tiles) pv(j - 1, pk);
        if (j < wave_tiles) qk(j, sc);
        block_barrier();
        const bool issues = j + 2 + grp < n_tiles;
        if (issues) issue(j + 2 + grp);
        if (j < wave_tiles) softmax(sc, row_max(j, sc), pk);
        if (issues) wait_all_but_newest(); else wait_vmem<0>();
        block_barrier();
      };
      general(0);
      const int j_ss = max(1, min(min(wave_tiles, first_masked), n_tiles - 3));
      int j = 1;
      for (; j < j_ss; ++j) {
        pv(j - 1, pk);
        qk(j, sc);
        block_barrier();
        issue(j + 2 + grp);
        softmax(sc, tile_max(sc), pk);
        wait_all_but_newest();
        block_barrier();
      }
      for (; j < n_tiles; ++j) general(j);
      finish(n_tiles - 1 < wave_tiles, pk);
    } else {
      // Block skip, in the same ping-pong, with the V load gated on the
      // decisions.  Waves w (group 0) and w+4 (group 1) hold the two halves
      // of one 64-row tile, and group 1 runs half an iteration behind.
      //  * Group 1, in its VALU phase j, reads group 0's votes on tile j
      //    (published in group 0's phase j, before the barrier), so it knows
      //    its tile's decision at once: a skipped tile loses its
      //    exponentials.  It copies V tile j when a group-0 half keeps it (a
      //    quarter per wave, as soon as the votes are read) or, failing
      //    that, when its own half does (the whole tile, from that wave).
      //    It waits for the copy at the end of its next MFMA phase, before
      //    either group's P.V of tile j.
      //  * Group 0 copies the K tiles (tile j+2 in its VALU phase j, into
      //    the stage of tile j-2), runs the exponentials of each live tile
      //    on which its own rows are not all negligible (such a tile is
      //    kept), and learns the decision on tile j from its partner's vote
      //    in its VALU phase j+1; the row sum of tile j waits until then
      //    (lpend) and is added, if the tile is kept, before that phase's
      //    rescale, which keeps the arithmetic of the dense kernel.  A tile
      //    kept only by the partner's half is recomputed then from K tile j,
      //    still in its stage.
      //  * P.V of tile j runs in MFMA phase j+2 for both groups (so the P of
      //    two tiles are held: pkA for even tiles, pkB for odd ones); V tile
      //    j overwrites tile j-4 in the V ring, whose last reader finished
      //    in MFMA phase j-2.  K tile j+2 overwrites tile j-2, read last by
      //    group 1's Q.K^T in the MFMA phase that ran beside group 0's VALU
      //    phase j-2 (and by group 0's recompute in its phase j-1).
      //  * The running max of the decisions (m_true) takes every tile,
      //    skipped or not.
      uint32_t pkA[2][8], pkB[2][8];
      int keepA = 0, keepB = 0;  // P.V due for the tile whose P is in pkA / pkB
      int mine_prev = 1, live_prev = 0;  // group 0: its vote on, and rows in, tile j-1
      int done_prev = 0;                 // group 0: the exponentials of tile j-1 were computed
      float lpend = 0.f;                 // group 0: row sum of tile j-1, added once it is kept
      block_barrier();
      if (grp == 1) block_barrier();
      // one phase pair; pk holds the P of tile j-2 (read in the MFMA phase)
      // and receives that of tile j; keep is the flag of that buffer's tile,
      // pko and keepo the other buffer and its flag.  STEADY: every step is
      // present and no mask is needed (the steady-state copy of the body).
      auto phase = [&](int j, uint32_t (*pk)[8], int& keep, uint32_t (*pko)[8], int& keepo,
                       auto steady_tag) {
        constexpr bool STEADY = decltype(steady_tag)::value;
        if (STEADY ? keep : (j >= 2 && keep)) pv(j - 2, pk);
        if (STEADY || j < wave_tiles) qk(j, sc);
        if (grp == 1) wait_vmem<0>();  // V tile j-1, before group 0's P.V of it
        block_barrier();
        apply_pending();
        const bool live = STEADY || j < wave_tiles;
        if (grp == 0) {
          const int pvote = j >= 1 ? read_partner(j - 1) : 1;
          int loads = 0;  // copies issued in this phase
          if (STEADY || j + 2 < n_tiles) {
            issue_k(j + 2, STEADY);
            loads = T::KPW;
          }
          float tmx = -INFINITY;
          int mine = 1;
          if (STEADY || j < n_tiles) {
            tmx = STEADY ? tile_max(sc) : (live ? row_max(j, sc) : -INFINITY);
            mine = vote_publish(j, tmx, live);
          }
          // tile j-1 decided: both halves negligible skips it
          keepo = live_prev & ((mine_prev & __builtin_amdgcn_readfirstlane(pvote)) ^ 1);
          if (keepo & done_prev) l += lpend;
          const float m_before = m_used;
          keep = live ? 1 : 0;  // for now; decided in the next phase
          lpend = 0.f;
          int done = 0;
          if (live && !mine) {
            rescale(tmx);
            lpend = exps(sc, pk, -m_used);
            done = 1;
          }
          if (keepo & (done_prev ^ 1)) {
            // Tile j-1 is kept although every row of this half was
            // negligible on it, so its exponentials were left out: its
            // scores are formed again from K tile j-1, still in LDS (a
            // 32-key half at a time), with the exponent reference of tile
            // j-1, and its row sum joins l scaled to the current reference.
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
              qk_half(j - 1, kb, sc[0]);
              if (!STEADY && j - 1 >= first_masked) {
                const int c0 = (j - 1) * BN + kb * 32, qi = q0 + n;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                  const int key = c0 + (i >> 2) * 8 + hf * 4 + (i & 3);
                  if (key >= S || key > off + qi) sc[0][i] = -INFINITY;
                }
              }
#pragma unroll
              for (int i = 0; i < 16; i += 2)
                pko[kb][i >> 1] = pack_bf16(fast_exp2(fmaf(sc[0][i], sl2, -m_before)),
                                            fast_exp2(fmaf(sc[0][i + 1], sl2, -m_before)));
#pragma unroll
              for (int i = 0; i < 8; ++i)
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pko[kb][i]), kOnes2, rs, false);
            }
            l += rs * fast_exp2(m_before - m_used);
          }
          mine_prev = mine;
          live_prev = live ? 1 : 0;
          done_prev = done;
          if (STEADY || j < n_tiles) m_true = fmaxf(m_true, tmx);
          if constexpr (STEADY) wait_vmem<T::KPW>(); else wait_vmem_upto(loads);
        } else if (STEADY || j < n_tiles) {
          const int v0 = read_votes0(j);
          const float tmx = STEADY ? tile_max(sc) : (live ? row_max(j, sc) : -INFINITY);
          const uint32_t negs0 = (uint32_t)__ballot(v0 != 0) & 0x0Fu;  // group 0's negligible halves
          const int keep0 = negs0 != 0x0Fu ? 1 : 0;                  // a group-0 half keeps tile j
          if (keep0) issue_v(j, STEADY);
          const int mine = vote_publish(j, tmx, live);
          const int sk = mine & (int)((negs0 >> kq) & 1u);
          keep = live ? sk ^ 1 : 0;
          if (keep) {
            softmax(sc, tmx, pk);
            if (!keep0) issue_v_all(j);  // only this half keeps V tile j
          }
          if (j < rec_tiles) record(j, sk);
          if (flush_due(j)) flush_skips(j & ~63);
          m_true = fmaxf(m_true, tmx);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the vote is in LDS before the barrier
        block_barrier();
      };
      using Gen = std::integral_constant<bool, false>;
      using Ste = std::integral_constant<bool, true>;
      // steady phases: 2 <= j < j_ss (P.V of j-2, Q.K^T of j, the copies of
      // K tile j+2 and V tile j, no mask, and neither the last tile, so
      // whole), run in pairs so that each P buffer stays in fixed registers
      const int j_ss = min(min(wave_tiles, first_masked), n_tiles - 4);
      phase(0, pkA, keepA, pkB, keepB, Gen{});
      if (1 <= n_tiles) phase(1, pkB, keepB, pkA, keepA, Gen{});
      int j = 2;
      for (; j + 1 < j_ss; j += 2) {
        phase(j, pkA, keepA, pkB, keepB, Ste{});
        phase(j + 1, pkB, keepB, pkA, keepA, Ste{});
      }
      for (; j <= n_tiles; j += 2) {
        phase(j, pkA, keepA, pkB, keepB, Gen{});
        if (j + 1 <= n_tiles) phase(j + 1, pkB, keepB, pkA, keepA, Gen{});
      }
      // MFMA phase n_tiles + 1: P.V of the last tile
      if ((n_tiles + 1) & 1) {
        if (keepB) pv(n_tiles - 1, pkB);
      } else {
        if (keepA) pv(n_tiles - 1, pkA);
      }
      finish(false, pkA);
    }

    if (!has_next()) break;
    prefetched = true;
    ring = (ring + n_tiles) % T::NST;
  }
}

template <int D, bool CAUSAL, bool SKIP, bool PAGED = false>
hipError_t launch_one(const Params& p, int grid, hipStream_t stream) {
  auto kern = prefill_bf16_kernel<D, CAUSAL, SKIP, PAGED>;
  constexpr size_t lds = Tile<D>::lds_bytes;
  static bool attr_set = false;  // per instantiation; idempotent if raced
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, p);
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
  const long long items = (long long)p.n_qblk * p.n_hgrp;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  p.n_items = (int)items;
  // Several items per workgroup hide an item's start and end behind its
  // neighbour's, as long as every compute unit still gets a workgroup (the
  // zigzag order balances pairs, so 1, 2 or 4).
  p.items_per_wg = a.skip ? 1 : p.n_items >= 4 * kComputeUnits ? 4 : p.n_items >= 2 * kComputeUnits ? 2 : 1;
  const int g = (p.n_items + p.items_per_wg - 1) / p.items_per_wg;
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

hipError_t launch_prefill_paged(const PagedPrefillArgs& a, hipStream_t stream) {
  Params p{};
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k_pool);
  p.v = static_cast<const uint16_t*>(a.v_pool);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.S = 0;
  p.G = a.Hq / a.Hkv;
  int gw = 8;
  while (p.G % gw) gw >>= 1;
  p.gw = gw;
  p.rows_per_wg = 32 * kWaves / gw;
  p.n_qblk = (a.max_seqlen_q + p.rows_per_wg - 1) / p.rows_per_wg;
  p.sub_per_kv = p.G / gw;
  p.n_hgrp = a.Hkv * p.sub_per_kv;
  p.sl2 = a.scale * 1.4426950408889634f;
  p.cu_q = a.cu_q;
  p.seq_k = a.seq_lens_k;
  p.table = a.block_table;
  p.N = a.N;
  p.max_blocks = a.max_blocks;
  p.num_blocks = a.num_blocks;
  p.total_q = a.total_q;
  p.max_seqlen_q = a.max_seqlen_q;
  const long long grid = (long long)p.n_qblk * a.N * p.n_hgrp;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const int g = (int)grid;
  p.n_items = g;
  p.items_per_wg = 1;
  return a.D == 64 ? launch_one<64, true, false, true>(p, g, stream)
                   : launch_one<128, true, false, true>(p, g, stream);
}

}  // namespace attn
