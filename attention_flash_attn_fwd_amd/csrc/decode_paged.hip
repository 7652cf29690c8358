// Paged-KV decode for gfx950: split-KV partial attention + log-sum-exp merge.
//
// One new query token per sequence attends to every cached token, whose K/V
// rows are found through a block table ("LLM推理优化技术综述" page,
// PageAttention part: the cache is cut into fixed-size blocks and a table maps
// a sequence's logical blocks to non-contiguous physical ones, like an OS
// page table; "TensorRT-LLM：大模型推理加速的工业级引擎", PagedAttention).
// Small-batch decode is bound by reading the KV cache from HBM (same page,
// decode stage), so the kernels are built around keeping K/V reads in flight:
//  * A workgroup is one wave and owns one (K/V head, 512-token split,
//    sequence).  The G = Hq/Hkv query heads of the K/V head are processed
//    together, so each K/V byte is read from HBM once (the GQA saving of the
//    "TensorRT对Grouped Query Attention的支持进展" page, 技术演进背景).  The
//    K/V head is the fastest grid index: the Hkv waves of one split run at
//    the same time and read the Hkv adjacent runs of each pool block, which
//    spreads the gather over more DRAM channels than scattered 4 KiB runs.
//  * Two pool layouts.  MFMA-native pools (decode_native_kernel) are read
//    straight into matrix-core operands; row-major pools ([block, head,
//    slot, dim], decode_split_kernel) are staged through LDS with
//    asynchronous 16-byte-per-lane DMA, double buffered, with the 16-byte
//    chunks of each row XOR-permuted so the operand reads are bank-conflict
//    free.
//  * S^T = K Q^T uses v_mfma_f32_16x16x32_bf16 with the query heads as the
//    16-wide N dimension (G <= 16); O^T += V^T P^T takes P^T straight from
//    the score accumulator.  Softmax is online, in base 2.
//  * The split's (O / l, log2-sum-exp) goes to the caller's workspace; the
//    merge kernel combines the splits: lse = log sum_s exp(lse_s),
//    O = sum_s exp(lse_s - lse) O_s.
#include "attn_internal.h"

#include <math.h>

#include <atomic>

#include "../../include/attn.h"

// Split-KV scratch of the allocation-free decode entry point: the partial
// outputs and log-sum-exps of one call, for callers that cannot allocate
// device memory.  Each GPU the library runs on holds one copy until the
// process ends.  Host code never passes this name to a kernel (on the host it
// is only a stand-in for the symbol): decode_static_scratch resolves the
// device address per GPU.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_STATIC_SCRATCH_BYTES];

namespace attn {

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_addr[kScratchDevices];
}  // namespace

hipError_t decode_static_scratch(int device, void** addr) {
  if (device < 0 || device >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[device].load(std::memory_order_acquire);
  if (p == nullptr) {
    // the caller made `device` current; every GPU has its own copy of the
    // array at its own address (racing first calls store the same value)
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[device].store(p, std::memory_order_release);
  }
  *addr = p;
  return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kBlk = 16;  // tokens per pool block
// Register budget of the split kernels: at least 3 resident waves per SIMD
// (<= 168 VGPRs for D = 128, no spills), so that the whole grid of a
// typical batch is resident at once and keeps enough K/V reads in flight.
constexpr int kDecodeWavesPerSimd = 3;
constexpr int kTT = 32;   // tokens per tile (two blocks)
constexpr float kUnset = -1e30f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

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
  int Hq, Hkv, G, num_blocks, max_blocks, n_split;
  float sl2;
  float v_scale;  // FP8 pools: V code -> value factor (1 otherwise)
  // block skip only
  float thr;                       // log2(lambda)
  uint8_t* skip_map;               // [N, Hkv, max_blocks] or null
  unsigned long long* skip_count;  // or null
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, b2));  // RNE
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes at gbase + voff land at LDS byte lds_addr + 16*i.  Issued
// from asm so that the compiler does not serialise it against unrelated LDS
// reads; completion is awaited explicitly with s_waitcnt vmcnt.  The load is
// non-temporal (nt): the K/V stream is read once and should not displace
// other lines from the caches.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               ::"v"(voff), "s"(gbase), "s"(m) : "memory");
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
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

// LDS tile: 32 rows (tokens) of D bf16, 16-byte chunk c of row r stored at
// slot c ^ swz(r).  K is read as 16-byte MFMA A fragments (16 rows, same
// chunk), V with the transposing 8-byte read (8 rows x 32 bytes per half
// wave); the XOR patterns spread both over all 64 banks.
template <int D>
struct DTile {
  static constexpr int RB = D * 2;             // bytes per row
  static constexpr int TB = kTT * RB;          // bytes per K (or V) tile
  static constexpr int NI = TB / 1024;         // DMA instructions per tensor per tile
  static constexpr int RPI = 1024 / RB;        // rows per DMA instruction
  static constexpr int NST = 2;                // stages (tiles resident or in flight)
  static constexpr int LDS = NST * 2 * TB;
  static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3); }
};

template <int D>
__global__ __launch_bounds__(64, kDecodeWavesPerSimd) void decode_split_kernel(DecParams p) {
  using T = DTile<D>;
  constexpr int NKS = D / 32;   // 32-dim k-steps of Q.K^T
  constexpr int NDB = D / 16;   // 16-dim output blocks of P.V
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[T::LDS];
  LDS_AS unsigned char* smem = (LDS_AS unsigned char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  const int kvh = blockIdx.x, split = blockIdx.y, n = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = lane & 15, g4 = lane >> 4;
  const int L = p.seq_lens[n];
  const int tok_begin = split * kDecodeSplitTokens;
  if (L <= 0 || tok_begin >= L) return;  // the merge kernel handles L <= 0
  const int n_tok = min(L - tok_begin, kDecodeSplitTokens);
  const int n_tiles = (n_tok + kTT - 1) / kTT;
  const int G = p.G;

  // The split's block-table entries, one per lane (lanes < n_blk), fetched
  // together with Q in a single round trip.  A bad entry or a length past
  // the table end poisons the whole sequence with NaN.
  const int32_t* trow = p.table + (size_t)n * p.max_blocks;
  const int lb0 = tok_begin / kBlk;
  const int n_blk = (n_tok + kBlk - 1) / kBlk;
  const bool in_table = lb0 + n_blk <= p.max_blocks;
  int my_ph = 0;
  if (in_table && lane < n_blk) my_ph = trow[lb0 + lane];
  // Q^T as the B operand: lane (head h, group g4) holds dims ks*32 + g4*8 .. +7
  bf16x8 qB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (h < G)
      qB[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)n * p.Hq + kvh * G + h) * D +
                                                ks * 32 + g4 * 8);
    else
      qB[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), visible to the compiler
  const bool lane_ok = lane >= n_blk || (my_ph >= 0 && my_ph < p.num_blocks);
  const bool bad = !in_table || !__all(lane_ok);
  const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
  if (bad) {
    if (h < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = f32x4{NAN, NAN, NAN, NAN};
      if (g4 == 0) p.ws_lse[slot] = NAN;
    }
    return;
  }

  const size_t head_stride = (size_t)kBlk * T::RB;             // bytes of one (block, head)
  const size_t blk_stride = (size_t)p.Hkv * head_stride;       // bytes of one pool block
  const unsigned char* kpool = reinterpret_cast<const unsigned char*>(p.k_pool) + kvh * head_stride;
  const unsigned char* vpool = reinterpret_cast<const unsigned char*>(p.v_pool) + kvh * head_stride;

  // DMA of tile t into stage t % NST.  Rows past the sequence end re-read its
  // last token, so every LDS row holds finite data (tail slots of the last
  // pool block may hold anything).
  auto issue = [&](int t) {
    const uint32_t st = smem_base + (t % T::NST) * 2 * T::TB;
    const int v = min(kTT, n_tok - t * kTT);   // valid rows of this tile
    const int ph0 = __builtin_amdgcn_readlane(my_ph, 2 * t);
    const int ph1 = v > kBlk ? __builtin_amdgcn_readlane(my_ph, 2 * t + 1) : ph0;
#pragma unroll
    for (int i = 0; i < T::NI; ++i) {
      const int row0 = i * T::RPI;
      const int bi = (row0 >= kBlk && v > kBlk) ? 1 : 0;   // block supplying these rows
      const int ph = bi ? ph1 : ph0;
      const int row = row0 + (lane * 16) / T::RB;
      const int slotc = ((lane * 16) % T::RB) / 16;
      const int src = min(row, v - 1) - bi * kBlk;          // row within the block
      const uint32_t ko = (uint32_t)src * T::RB + ((slotc ^ T::swz_k(row)) << 4);
      const uint32_t vo = (uint32_t)src * T::RB + ((slotc ^ T::swz_v(row)) << 4);
      dma16(kpool + (size_t)ph * blk_stride, ko, st + i * 1024);
      dma16(vpool + (size_t)ph * blk_stride, vo, st + T::TB + i * 1024);
    }
  };

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = kUnset, l = 0.f;
  const float sl2 = p.sl2;
  // per-lane LDS offsets: K fragment (row h of block b, chunk 4ks + g4);
  // V^T fragment source (rows base + s/4, dims d0 + 4(s%4))
  const int vs = lane & 15;
  const int v_row0 = 4 * g4 + (vs >> 2);

  for (int t = 0; t < min(n_tiles, T::NST - 1); ++t) issue(t);
  // wait until tile t has landed, given how many later tiles are in flight
  auto wait_tile = [&](int later) {
    switch (later) {
      case 0: wait_vmem<0>(); break;
      case 1: wait_vmem<2 * T::NI>(); break;
      case 2: wait_vmem<4 * T::NI>(); break;
      default: wait_vmem<6 * T::NI>(); break;
    }
  };
  for (int t = 0; t < n_tiles; ++t) {
    // stage (t-1) % NST was fully read at the end of the previous iteration
    if (t + T::NST - 1 < n_tiles) issue(t + T::NST - 1);
    wait_tile(min(t + T::NST - 1, n_tiles - 1) - t);
    asm volatile("" ::: "memory");
    const LDS_AS unsigned char* kl = smem + (t % T::NST) * 2 * T::TB;
    const LDS_AS unsigned char* vl = kl + T::TB;

    // scores S^T (32 tokens x 16 heads): lane (h, g4) gets tokens b*16 + 4*g4 + i
    f32x4 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = b * 16 + h;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = 4 * ks + g4;
        const bf16x8 a =
            *reinterpret_cast<const LDS_AS bf16x8*>(kl + row * T::RB + ((c ^ T::swz_k(row)) << 4));
        s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qB[ks], s[b], 0, 0, 0);
      }
    }
    const int valid = n_tok - t * kTT;
    if (valid < kTT) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (b * 16 + 4 * g4 + i >= valid) s[b][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    const float tmx = half_swap_max(mx) * sl2;
    if (__any(tmx > m_used + 8.f)) {  // lazy rescale (exponent reference moves by > 2^8)
      const float m_new = fmaxf(m_used, tmx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float nm = -m_used;
    // packed bf16 P^T (B operand): slots j<4 are tokens 4*g4+j of block 0,
    // slots j>=4 tokens 4*g4+j-4 of block 1.  Kept as a plain array: the
    // row-sum dot products below must see the four words separately.
    uint32_t pk[4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      pk[2 * b] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[b][0], sl2, nm)),
                            __builtin_amdgcn_exp2f(fmaf(s[b][1], sl2, nm)));
      pk[2 * b + 1] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[b][2], sl2, nm)),
                                __builtin_amdgcn_exp2f(fmaf(s[b][3], sl2, nm)));
    }
    float rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[0]), kOnes2, 0.f, false);
    float rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[1]), kOnes2, 0.f, false);
    rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[2]), kOnes2, rs0, false);
    rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[3]), kOnes2, rs1, false);
    l += rs0 + rs1;
    const u32x4 pw = {pk[0], pk[1], pk[2], pk[3]};
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    // O^T += V^T P^T: V^T rows d = db*16 + lane%16, token slots 8*g4 + j
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + 4 * (vs & 3);
      const int c = d >> 3;
      const int r0 = v_row0, r1 = 16 + v_row0;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS s16x4*)(vl + r0 * T::RB + ((c ^ T::swz_v(r0)) << 4) + (d & 7) * 2));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS s16x4*)(vl + r1 * T::RB + ((c ^ T::swz_v(r1)) << 4) + (d & 7) * 2));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[db], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage t fully read
  }

  // combine the four lanes of each head and write the split's partial result
  float lt = l + __shfl_xor(l, 16);
  lt = half_swap_add(lt);
  if (h < G) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = acc[db] * inv;
    if (g4 == 0) p.ws_lse[slot] = m_used + __log2f(lt);
  }
}

// Decode over a pool in the MFMA-native layout: inside each (block, head)
// run, K is stored as 8-element chunks, chunk-major ([D/8][16][8]), and V is
// stored transposed ([D][16]).  Every MFMA operand is then one plain vector
// load from HBM with no LDS staging:
//  * S^T = K Q^T (v_mfma_f32_16x16x32_bf16): lane (token t = lane%16,
//    group g = lane/16) loads chunk 4*ks + g of token t, 16 bytes; the 64
//    lanes of one load cover 1 KiB contiguously.
//  * O^T += V^T P^T (v_mfma_f32_16x16x16_bf16): lane (dim d = lane%16 +
//    16*db, group g) loads V^T[d][4g .. 4g+3], 8 bytes; 512 contiguous bytes
//    per load.  Its k-slots are exactly the keys the S^T accumulator gives
//    the same lane, so P^T needs no shuffle.
// Loads run two blocks ahead of the MFMAs; occupancy is high because no LDS
// is used, which keeps many K/V bytes in flight.  K/V are read once per
// call, so the loads are non-temporal: the stream does not evict other
// lines from L2 and the last-level cache (this alone raised the gather rate
// from about 4.8 to 5.5 TB/s).
template <int D>
__global__ __launch_bounds__(64, kDecodeWavesPerSimd) void decode_native_kernel(DecParams p) {
  constexpr int NKS = D / 32;  // 32-dim k-steps of Q.K^T
  constexpr int NDB = D / 16;  // 16-dim output blocks of P.V
  constexpr int RUN = kBlk * D * 2;  // bytes of one (block, head) run

  const int kvh = blockIdx.x, split = blockIdx.y, n = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = lane & 15, g4 = lane >> 4;
  const int L = p.seq_lens[n];
  const int tok_begin = split * kDecodeSplitTokens;
  if (L <= 0 || tok_begin >= L) return;  // the merge kernel handles L <= 0
  const int n_tok = min(L - tok_begin, kDecodeSplitTokens);
  const int G = p.G;

  const int32_t* trow = p.table + (size_t)n * p.max_blocks;
  const int lb0 = tok_begin / kBlk;
  const int n_blk = (n_tok + kBlk - 1) / kBlk;
  const bool in_table = lb0 + n_blk <= p.max_blocks;
  int my_ph = 0;
  if (in_table && lane < n_blk) my_ph = trow[lb0 + lane];
  bf16x8 qB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (h < G)
      qB[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)n * p.Hq + kvh * G + h) * D +
                                                ks * 32 + g4 * 8);
    else
      qB[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const bool lane_ok = lane >= n_blk || (my_ph >= 0 && my_ph < p.num_blocks);
  const bool bad = !in_table || !__all(lane_ok);
  const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
  if (bad) {
    if (h < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = f32x4{NAN, NAN, NAN, NAN};
      if (g4 == 0) p.ws_lse[slot] = NAN;
    }
    return;
  }

  const size_t blk_stride = (size_t)p.Hkv * RUN;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k_pool) + (size_t)kvh * RUN;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v_pool) + (size_t)kvh * RUN;
  const uint32_t k_off = (uint32_t)((g4 * 16 + h) * 16);       // + ks * 1024
  const uint32_t v_off = (uint32_t)((h * 16 + 4 * g4) * 2);    // + db * 512

  struct Buf {
    bf16x8 k[NKS];
    s16x4 v[NDB];
  };
  auto load = [&](int j, Buf& b) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(my_ph, j);
    const unsigned char* kb = kbase + ph * blk_stride + k_off;
    const unsigned char* vb = vbase + ph * blk_stride + v_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      b.k[ks] = __builtin_bit_cast(
          bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + ks * 1024)));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      b.v[db] = __builtin_bit_cast(
          s16x4, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + db * 512)));
  };

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = kUnset, l = 0.f;
  const float sl2 = p.sl2;

  auto compute = [&](int j, Buf& b) {
    // scores S^T (16 tokens x 16 heads): lane (h, g4) gets tokens 4*g4 + i
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b.k[ks], qB[ks], s, 0, 0, 0);
    const int valid = n_tok - j * kBlk;
    if (valid < kBlk) {
      // slots past the sequence end: no score, and their V (arbitrary bits,
      // possibly NaN) must not reach P.V, where 0 * NaN would poison O
      uint32_t keep[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g4 + i >= valid) s[i] = -INFINITY;
      keep[0] = (4 * g4 + 0 < valid ? 0xffffu : 0u) | (4 * g4 + 1 < valid ? 0xffff0000u : 0u);
      keep[1] = (4 * g4 + 2 < valid ? 0xffffu : 0u) | (4 * g4 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x2 w = __builtin_bit_cast(u32x2, b.v[db]);
        w[0] &= keep[0];
        w[1] &= keep[1];
        b.v[db] = __builtin_bit_cast(s16x4, w);
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    const float tmx = half_swap_max(mx) * sl2;
    if (__any(tmx > m_used + 8.f)) {  // lazy rescale (exponent reference moves by > 2^8)
      const float m_new = fmaxf(m_used, tmx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float nm = -m_used;
    const uint32_t pk0 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[0], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[1], sl2, nm)));
    const uint32_t pk1 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[2], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[3], sl2, nm)));
    l += __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), kOnes2, 0.f, false) +
         __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), kOnes2, 0.f, false);
    const u32x2 pw = {pk0, pk1};
    const s16x4 pB = __builtin_bit_cast(s16x4, pw);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(b.v[db], pB, acc[db], 0, 0, 0);
  };

  // two buffers, loads two blocks ahead of the MFMAs
  Buf b0, b1;
  load(0, b0);
  if (n_blk > 1) load(1, b1);
  for (int j = 0; j < n_blk; j += 2) {
    compute(j, b0);
    if (j + 2 < n_blk) load(j + 2, b0);
    if (j + 1 < n_blk) {
      compute(j + 1, b1);
      if (j + 3 < n_blk) load(j + 3, b1);
    }
  }

  float lt = l + __shfl_xor(l, 16);
  lt = half_swap_add(lt);
  if (h < G) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = acc[db] * inv;
    if (g4 == 0) p.ws_lse[slot] = m_used + __log2f(lt);
  }
}

// Decode over an FP8 (E4M3) pool with one scale per pool (a quantised KV
// cache: "TensorRT-LLM：大模型推理加速的工业级引擎", 六大核心优化技术 / 量化
// lists FP8, and its 深入版解读 names the E4M3/E5M2 encodings; decode time is
// the KV-cache read from HBM, which FP8 halves).  The pool keeps each
// (block, head) run in an MFMA-native byte order (16 * D bytes):
//  * K: 16-byte chunks of 16 dims; chunk c of token t at
//    (c / 4) * 1024 + ((c % 4) * 16 + t) * 16.  Lane (t = lane % 16, g =
//    lane / 16) loads 16 bytes at i * 1024 + lane * 16 (1 KiB contiguous per
//    load): dims (4i + g) * 16 .. +15 of token t, which become the A
//    fragments of two 8-dim k-steps; Q^T is loaded with the same dims.
//  * V: for 16-dim block b and token t, the byte of dim b * 16 + r sits at
//    (b / 4) * 1024 + ((t / 4) * 16 + r) * 16 + (b % 4) * 4 + t % 4, so the
//    16 bytes of lane (r, g) hold, per block b, the four tokens 4g .. 4g+3
//    that the 16x16x16 MFMA takes from it (again 1 KiB per load).
// Codes are widened to bf16 exactly (every E4M3 value is a bf16 value) by
// the pair conversion; the K scale is folded into the softmax scale and the
// V scale into the final 1 / l, both in fp32.  Loads run NBUF blocks ahead;
// two is fastest (more gathers in flight per wave measured slower: 4, 8 and
// 16 blocks ahead took 10%, 14% and 95% longer).
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t w) {
  // codes of bytes 0-1 (HI = false) or 2-3 as two bf16; the pair is used as
  // one 32-bit word (its halves are never extracted one by one)
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

template <int D, int NBUF>
__global__ __launch_bounds__(64, kDecodeWavesPerSimd) void decode_fp8_kernel(DecParams p) {
  constexpr int NKS = D / 32;   // 32-dim k-steps of Q.K^T
  constexpr int NDB = D / 16;   // 16-dim output blocks of P.V
  constexpr int NI = D / 64;    // 1 KiB loads per block, K and V each
  constexpr int RUN = kBlk * D; // bytes of one (block, head) run

  const int kvh = blockIdx.x, split = blockIdx.y, n = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = lane & 15, g4 = lane >> 4;
  const int L = p.seq_lens[n];
  const int tok_begin = split * kDecodeSplitTokens;
  if (L <= 0 || tok_begin >= L) return;  // the merge kernel handles L <= 0
  const int n_tok = min(L - tok_begin, kDecodeSplitTokens);
  const int G = p.G;

  const int32_t* trow = p.table + (size_t)n * p.max_blocks;
  const int lb0 = tok_begin / kBlk;
  const int n_blk = (n_tok + kBlk - 1) / kBlk;
  const bool in_table = lb0 + n_blk <= p.max_blocks;
  int my_ph = 0;
  if (in_table && lane < n_blk) my_ph = trow[lb0 + lane];
  // Q^T fragment of k-step 2i + j: dims (g4 + 4i) * 16 + j * 8 .. +7
  bf16x8 qB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (h < G)
      qB[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)n * p.Hq + kvh * G + h) * D +
                                                (g4 + 4 * (ks >> 1)) * 16 + (ks & 1) * 8);
    else
      qB[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const bool lane_ok = lane >= n_blk || (my_ph >= 0 && my_ph < p.num_blocks);
  const bool bad = !in_table || !__all(lane_ok);
  const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
  if (bad) {
    if (h < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = f32x4{NAN, NAN, NAN, NAN};
      if (g4 == 0) p.ws_lse[slot] = NAN;
    }
    return;
  }

  const size_t blk_stride = (size_t)p.Hkv * RUN;
  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(p.k_pool) + (size_t)kvh * RUN + lane * 16;
  const unsigned char* vbase =
      reinterpret_cast<const unsigned char*>(p.v_pool) + (size_t)kvh * RUN + lane * 16;

  struct Buf {
    u32x4 k[NI];
    u32x4 v[NI];
  };
  auto load = [&](int j, Buf& b) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(my_ph, j);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      b.k[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + ph * blk_stride + i * 1024));
      b.v[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(vbase + ph * blk_stride + i * 1024));
    }
  };

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = kUnset, l = 0.f;
  const float sl2 = p.sl2;

  auto compute = [&](int j, const Buf& b) {
    // scores S^T (16 tokens x 16 heads): lane (h, g4) gets tokens 4*g4 + i
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const uint32_t w0 = b.k[i][2 * jj], w1 = b.k[i][2 * jj + 1];
        const u32x4 kw = {fp8_pair<false>(w0), fp8_pair<true>(w0), fp8_pair<false>(w1),
                          fp8_pair<true>(w1)};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw),
                                                    qB[2 * i + jj], s, 0, 0, 0);
      }
    // slots past the sequence end: no score, and a zero code (+0) for their
    // V (the bytes there may be anything, NaN codes included).  Branch-free,
    // so no read of the MFMA result follows a branch.
    const int valid = n_tok - j * kBlk;
    uint32_t vkeep = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = 4 * g4 + i < valid;
      s[i] = ok ? s[i] : -INFINITY;
      vkeep |= ok ? (0xffu << (8 * i)) : 0u;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    const float tmx = half_swap_max(mx) * sl2;
    if (__any(tmx > m_used + 8.f)) {  // lazy rescale (exponent reference moves by > 2^8)
      const float m_new = fmaxf(m_used, tmx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float nm = -m_used;
    const uint32_t pk0 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[0], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[1], sl2, nm)));
    const uint32_t pk1 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[2], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[3], sl2, nm)));
    l += __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), kOnes2, 0.f, false) +
         __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), kOnes2, 0.f, false);
    const u32x2 pw = {pk0, pk1};
    const s16x4 pB = __builtin_bit_cast(s16x4, pw);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint32_t w = b.v[db >> 2][db & 3] & vkeep;
      const u32x2 vw = {fp8_pair<false>(w), fp8_pair<true>(w)};
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vw), pB,
                                                          acc[db], 0, 0, 0);
    }
  };

  // NBUF buffers with fixed registers, loads NBUF blocks ahead
  Buf buf[NBUF];
#pragma unroll
  for (int u = 0; u < NBUF; ++u)
    if (u < n_blk) load(u, buf[u]);
  for (int j = 0; j < n_blk; j += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      if (j + u < n_blk) {
        compute(j + u, buf[u]);
        if (j + u + NBUF < n_blk) load(j + u + NBUF, buf[u]);
      }
    }
  }

  float lt = l + __shfl_xor(l, 16);
  lt = half_swap_add(lt);
  if (h < G) {
    const float inv = p.v_scale / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = acc[db] * inv;
    if (g4 == 0) p.ws_lse[slot] = m_used + __log2f(lt);
  }
}

// Decode with block skipping ("高效部署稀疏注意力加速方案：BLASST方法详解与实践
// 指南", 架构与组件: blocks whose scores are negligible next to the running
// maximum of the blockwise online softmax lose their exp, their V load and
// their matrix product), on MFMA-native pools.  Inside a split the pool
// blocks are walked in order; for every query head h of the K/V group the
// block maximum tm_h is compared with the running maximum m_h of the
// split's earlier blocks, and the block is skipped when tm_h - m_h < log2
// lambda for all h (the V block is shared by the group).  The split's first
// block is always kept.  The V load is the decode's cost, so it is issued
// only after the decision: K runs two blocks ahead, the block's scores and
// decision come next, its V is loaded if kept and consumed one step later.
// The loop is unrolled six times so that the three K and two V buffers have
// fixed registers (moving a register whose load is in flight would wait).
template <int D>
__global__ __launch_bounds__(64, kDecodeWavesPerSimd) void decode_skip_kernel(DecParams p) {
  constexpr int NKS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int RUN = kBlk * D * 2;

  const int kvh = blockIdx.x, split = blockIdx.y, n = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = lane & 15, g4 = lane >> 4;
  const int L = p.seq_lens[n];
  const int tok_begin = split * kDecodeSplitTokens;
  if (L <= 0 || tok_begin >= L) return;
  const int n_tok = min(L - tok_begin, kDecodeSplitTokens);
  const int G = p.G;

  const int32_t* trow = p.table + (size_t)n * p.max_blocks;
  const int lb0 = tok_begin / kBlk;
  const int n_blk = (n_tok + kBlk - 1) / kBlk;
  const bool in_table = lb0 + n_blk <= p.max_blocks;
  int my_ph = 0;
  if (in_table && lane < n_blk) my_ph = trow[lb0 + lane];
  bf16x8 qB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (h < G)
      qB[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)n * p.Hq + kvh * G + h) * D +
                                                ks * 32 + g4 * 8);
    else
      qB[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  const bool lane_ok = lane >= n_blk || (my_ph >= 0 && my_ph < p.num_blocks);
  const bool bad = !in_table || !__all(lane_ok);
  const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
  if (bad) {
    if (h < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = f32x4{NAN, NAN, NAN, NAN};
      if (g4 == 0) p.ws_lse[slot] = NAN;
    }
    return;
  }

  const size_t blk_stride = (size_t)p.Hkv * RUN;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k_pool) + (size_t)kvh * RUN;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v_pool) + (size_t)kvh * RUN;
  const uint32_t k_off = (uint32_t)((g4 * 16 + h) * 16);
  const uint32_t v_off = (uint32_t)((h * 16 + 4 * g4) * 2);
  auto load_k = [&](int j, bf16x8* kb) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(my_ph, j);
    const unsigned char* src = kbase + ph * blk_stride + k_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kb[ks] = __builtin_bit_cast(
          bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ks * 1024)));
  };
  auto load_v = [&](int j, s16x4* vb) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(my_ph, j);
    const unsigned char* src = vbase + ph * blk_stride + v_off;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vb[db] = __builtin_bit_cast(
          s16x4, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src + db * 512)));
  };

  const float sl2 = p.sl2;
  // raw scores S^T of block j (tail slots -inf) and their per-head maximum
  auto scores = [&](int j, const bf16x8* kb) -> f32x4 {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks], qB[ks], s, 0, 0, 0);
    // branch-free tail mask: the first reads of the MFMA result stay in the
    // MFMA's basic block, where the compiler counts the wait states a VALU
    // read of an MFMA result needs (across a branch they were not counted)
    const int valid = n_tok - j * kBlk;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = 4 * g4 + i < valid ? s[i] : -INFINITY;
    return s;
  };
  auto block_max = [&](const f32x4& s) -> float {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    return half_swap_max(mx) * sl2;
  };

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = kUnset, l = 0.f;
  float m_true = kUnset;  // running max of the split's earlier blocks (log2 units)
  unsigned skipped = 0;
  // skip decision for block j (j = 0 is the split's first block: kept)
  auto decide = [&](int j, float tmx) -> bool {
    bool neg = true;  // padding columns (h >= G) never keep a block
    if (h < G) neg = m_true > 0.5f * kUnset && tmx - m_true < p.thr;
    const bool sk = j > 0 && __all(neg);
    m_true = fmaxf(m_true, tmx);
    if (lane == 0 && p.skip_map)
      p.skip_map[((size_t)n * p.Hkv + kvh) * p.max_blocks + lb0 + j] = sk ? 1 : 0;
    skipped += sk ? 1u : 0u;
    return sk;
  };
  // softmax and O^T += V^T P^T of a kept block
  auto finish = [&](int j, f32x4 s, float tmx, s16x4* vb) {
    const int valid = n_tok - j * kBlk;
    if (valid < kBlk) {
      uint32_t keep[2];
      keep[0] = (4 * g4 + 0 < valid ? 0xffffu : 0u) | (4 * g4 + 1 < valid ? 0xffff0000u : 0u);
      keep[1] = (4 * g4 + 2 < valid ? 0xffffu : 0u) | (4 * g4 + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x2 w = __builtin_bit_cast(u32x2, vb[db]);
        w[0] &= keep[0];
        w[1] &= keep[1];
        vb[db] = __builtin_bit_cast(s16x4, w);
      }
    }
    if (__any(tmx > m_used + 8.f)) {
      const float m_new = fmaxf(m_used, tmx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float nm = -m_used;
    const uint32_t pk0 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[0], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[1], sl2, nm)));
    const uint32_t pk1 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[2], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[3], sl2, nm)));
    l += __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), kOnes2, 0.f, false) +
         __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), kOnes2, 0.f, false);
    const u32x2 pw = {pk0, pk1};
    const s16x4 pB = __builtin_bit_cast(s16x4, pw);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb[db], pB, acc[db], 0, 0, 0);
  };

  bf16x8 k0[NKS], k1[NKS], k2[NKS];
  s16x4 v0[NDB], v1[NDB];
  f32x4 s_cur;
  float t_cur;
  bool keep_cur;
  // step j: score and decide block j+1 (its K has arrived), load its V if
  // kept and the K of block j+3 into the buffer block j used; then finish
  // block j with the V loaded one step earlier
  auto step = [&](int j, const bf16x8* ksc, bf16x8* kld, s16x4* vcur, s16x4* vnxt) {
    f32x4 s_n = {0.f, 0.f, 0.f, 0.f};
    float t_n = 0.f;
    bool keep_n = false;
    if (j + 1 < n_blk) {
      s_n = scores(j + 1, ksc);
      t_n = block_max(s_n);
      keep_n = !decide(j + 1, t_n);
      if (keep_n) load_v(j + 1, vnxt);
      if (j + 3 < n_blk) load_k(j + 3, kld);
    }
    if (keep_cur) finish(j, s_cur, t_cur, vcur);
    s_cur = s_n;
    t_cur = t_n;
    keep_cur = keep_n;
  };
  load_k(0, k0);
  if (n_blk > 1) load_k(1, k1);
  s_cur = scores(0, k0);
  t_cur = block_max(s_cur);
  keep_cur = !decide(0, t_cur);
  load_v(0, v0);
  if (n_blk > 2) load_k(2, k2);
  for (int j = 0; j < n_blk; j += 6) {
    step(j, k1, k0, v0, v1);
    if (j + 1 >= n_blk) break;
    step(j + 1, k2, k1, v1, v0);
    if (j + 2 >= n_blk) break;
    step(j + 2, k0, k2, v0, v1);
    if (j + 3 >= n_blk) break;
    step(j + 3, k1, k0, v1, v0);
    if (j + 4 >= n_blk) break;
    step(j + 4, k2, k1, v0, v1);
    if (j + 5 >= n_blk) break;
    step(j + 5, k0, k2, v1, v0);
  }

  if (lane == 0 && skipped && p.skip_count)
    atomicAdd(p.skip_count, (unsigned long long)skipped);
  float lt = l + __shfl_xor(l, 16);
  lt = half_swap_add(lt);
  if (h < G) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = acc[db] * inv;
    if (g4 == 0) p.ws_lse[slot] = m_used + __log2f(lt);
  }
}

// The same block skip on row-major pools ([block, head, slot, dim]), so one
// cache layout serves the dense decode, the block-skip decode and the
// chunked prefill.  K comes straight into operand registers (lane (h, g4)
// reads 16 bytes of token h's row per 32-dim step); a kept block's V rows
// are copied into an LDS stage (asynchronous 16-byte-per-lane copy, chunks
// XOR-permuted as in the split kernel) and read back transposed.  The order
// of one step is that of the MFMA-native kernel: score and decide block j+1,
// copy its V if kept, load the K of block j+3, then finish block j once its
// V copy (issued one step earlier) has landed.
template <int D>
__global__ __launch_bounds__(64, kDecodeWavesPerSimd) void decode_skip_rm_kernel(DecParams p) {
  using T = DTile<D>;
  constexpr int NKS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int RB = D * 2;               // bytes of one token row
  constexpr int RUN = kBlk * RB;          // bytes of one (block, head)
  constexpr int NVI = RUN / 1024;         // copy instructions per V block
  constexpr int RPI = 1024 / RB;          // rows per copy instruction
  __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[2 * RUN];
  LDS_AS unsigned char* smem = (LDS_AS unsigned char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  const int kvh = blockIdx.x, split = blockIdx.y, n = blockIdx.z;
  const int lane = threadIdx.x;
  const int h = lane & 15, g4 = lane >> 4;
  const int L = p.seq_lens[n];
  const int tok_begin = split * kDecodeSplitTokens;
  if (L <= 0 || tok_begin >= L) return;
  const int n_tok = min(L - tok_begin, kDecodeSplitTokens);
  const int G = p.G;

  const int32_t* trow = p.table + (size_t)n * p.max_blocks;
  const int lb0 = tok_begin / kBlk;
  const int n_blk = (n_tok + kBlk - 1) / kBlk;
  const bool in_table = lb0 + n_blk <= p.max_blocks;
  int my_ph = 0;
  if (in_table && lane < n_blk) my_ph = trow[lb0 + lane];
  bf16x8 qB[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (h < G)
      qB[ks] = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)n * p.Hq + kvh * G + h) * D +
                                                ks * 32 + g4 * 8);
    else
      qB[ks] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), visible to the compiler
  const bool lane_ok = lane >= n_blk || (my_ph >= 0 && my_ph < p.num_blocks);
  const bool bad = !in_table || !__all(lane_ok);
  const size_t slot = ((size_t)n * p.Hq + kvh * G + h) * p.n_split + split;
  if (bad) {
    if (h < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = f32x4{NAN, NAN, NAN, NAN};
      if (g4 == 0) p.ws_lse[slot] = NAN;
    }
    return;
  }

  const size_t blk_stride = (size_t)p.Hkv * RUN;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k_pool) + (size_t)kvh * RUN;
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(p.v_pool) + (size_t)kvh * RUN;
  const uint32_t k_off = (uint32_t)(h * RB + g4 * 16);  // + ks * 64
  auto load_k = [&](int j, bf16x8* kb) {
    const size_t ph = (size_t)__builtin_amdgcn_readlane(my_ph, j);
    const unsigned char* src = kbase + ph * blk_stride + k_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kb[ks] = __builtin_bit_cast(
          bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ks * 64)));
  };
  // V rows of block j into LDS stage j % 2; rows past the sequence end
  // re-read its last token, so every row holds finite data
  auto copy_v = [&](int j) {
    const int ph = __builtin_amdgcn_readlane(my_ph, j);
    const int valid = min(kBlk, n_tok - j * kBlk);
    const uint32_t st = smem_base + (j & 1) * RUN;
#pragma unroll
    for (int i = 0; i < NVI; ++i) {
      const int row = i * RPI + (lane * 16) / RB;
      const int slotc = ((lane * 16) % RB) / 16;
      const uint32_t vo = (uint32_t)min(row, valid - 1) * RB + ((slotc ^ T::swz_v(row)) << 4);
      dma16(vbase + (size_t)ph * blk_stride, vo, st + i * 1024);
    }
  };

  const float sl2 = p.sl2;
  auto scores = [&](int j, const bf16x8* kb) -> f32x4 {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks], qB[ks], s, 0, 0, 0);
    // branch-free tail mask (see decode_skip_kernel)
    const int valid = n_tok - j * kBlk;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = 4 * g4 + i < valid ? s[i] : -INFINITY;
    return s;
  };
  auto block_max = [&](const f32x4& s) -> float {
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    return half_swap_max(mx) * sl2;
  };

  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_used = kUnset, l = 0.f;
  float m_true = kUnset;  // running max of the split's earlier blocks (log2 units)
  unsigned skipped = 0;
  auto decide = [&](int j, float tmx) -> bool {
    bool neg = true;  // padding columns (h >= G) never keep a block
    if (h < G) neg = m_true > 0.5f * kUnset && tmx - m_true < p.thr;
    const bool sk = j > 0 && __all(neg);
    m_true = fmaxf(m_true, tmx);
    if (lane == 0 && p.skip_map)
      p.skip_map[((size_t)n * p.Hkv + kvh) * p.max_blocks + lb0 + j] = sk ? 1 : 0;
    skipped += sk ? 1u : 0u;
    return sk;
  };
  // V^T fragment of dims db*16 + lane%16, tokens 4*g4 .. +3: transposing
  // read of rows 4*g4 + (lane%16)/4, dims db*16 + 4*(lane%4) .. +3
  const int vs = lane & 15;
  const int v_row = 4 * g4 + (vs >> 2);
  auto finish = [&](int j, f32x4 s, float tmx) {
    const LDS_AS unsigned char* vl = smem + (j & 1) * RUN;
    if (__any(tmx > m_used + 8.f)) {
      const float m_new = fmaxf(m_used, tmx);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_used = m_new;
    }
    const float nm = -m_used;
    const uint32_t pk0 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[0], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[1], sl2, nm)));
    const uint32_t pk1 = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[2], sl2, nm)),
                                   __builtin_amdgcn_exp2f(fmaf(s[3], sl2, nm)));
    l += __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk0), kOnes2, 0.f, false) +
         __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk1), kOnes2, 0.f, false);
    const u32x2 pw = {pk0, pk1};
    const s16x4 pB = __builtin_bit_cast(s16x4, pw);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + 4 * (vs & 3);
      const int c = d >> 3;
      const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS s16x4*)(vl + v_row * RB + ((c ^ T::swz_v(v_row)) << 4) + (d & 7) * 2));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pB, acc[db], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage read before it is refilled
  };

  bf16x8 k0[NKS], k1[NKS], k2[NKS];
  f32x4 s_cur;
  float t_cur;
  bool keep_cur;
  // step j: score and decide block j+1 (its K has arrived), copy its V if
  // kept and load the K of block j+3 into the buffer block j used; then
  // finish block j once the V copy issued one step earlier has landed (the
  // operations issued after it are counted: those copies and loads)
  auto step = [&](int j, const bf16x8* ksc, bf16x8* kld) {
    f32x4 s_n = {0.f, 0.f, 0.f, 0.f};
    float t_n = 0.f;
    bool keep_n = false;
    int later = j + 2 < n_blk ? NKS : 0;  // K of block j+2, loaded last step
    if (j + 1 < n_blk) {
      s_n = scores(j + 1, ksc);
      t_n = block_max(s_n);
      keep_n = !decide(j + 1, t_n);
      if (keep_n) {
        copy_v(j + 1);
        later += NVI;
      }
      if (j + 3 < n_blk) {
        load_k(j + 3, kld);
        later += NKS;
      }
    }
    if (keep_cur) {
      wait_vmem_upto(later);
      finish(j, s_cur, t_cur);
    }
    s_cur = s_n;
    t_cur = t_n;
    keep_cur = keep_n;
  };
  load_k(0, k0);
  if (n_blk > 1) load_k(1, k1);
  s_cur = scores(0, k0);
  t_cur = block_max(s_cur);
  keep_cur = !decide(0, t_cur);
  copy_v(0);
  if (n_blk > 2) load_k(2, k2);
  for (int j = 0; j < n_blk; j += 3) {
    step(j, k1, k0);
    if (j + 1 >= n_blk) break;
    step(j + 1, k2, k1);
    if (j + 2 >= n_blk) break;
    step(j + 2, k0, k2);
  }

  if (lane == 0 && skipped && p.skip_count)
    atomicAdd(p.skip_count, (unsigned long long)skipped);
  float lt = l + __shfl_xor(l, 16);
  lt = half_swap_add(lt);
  if (h < G) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(p.ws_o + slot * D + db * 16 + 4 * g4) = acc[db] * inv;
    if (g4 == 0) p.ws_lse[slot] = m_used + __log2f(lt);
  }
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v = {x, 0.f};
  return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2)) & 0xffffu);
}

// One wave per (query head, sequence).  The lanes own splits while the
// weights are formed (max and sum are wave reductions), then own D/64
// output dims each while the weighted partial outputs are summed.  The
// sequence length, the first 64 splits' log-sum-exps and the first CH
// splits' partial outputs do not depend on each other, so they are loaded
// together before anything is decided (one memory round trip for up to CH
// splits); workspace slots past the sequence's splits hold stale values
// and are only ever selected away, never multiplied.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecParams p) {
  constexpr int DPL = D / 64;  // output dims per lane
  constexpr int CH = 8;        // splits whose partial outputs are loaded at once
  const int h = blockIdx.x, n = blockIdx.y, lane = threadIdx.x;
  const size_t out = (size_t)n * p.Hq + h;
  uint16_t* orow = p.o + out * D + lane * DPL;
  const float* lse_s = p.ws_lse + out * p.n_split;
  const float* o_s = p.ws_o + out * p.n_split * D + lane * DPL;
  const int L = p.seq_lens[n];
  const float lse0 = lane < p.n_split ? lse_s[lane] : kUnset;
  float part[CH][DPL];
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < DPL; ++e) part[c][e] = c < p.n_split ? o_s[(size_t)c * D + e] : 0.f;
  if (L <= 0 || (long long)L > (long long)p.max_blocks * kBlk) {
    const uint16_t fill = L == 0 ? 0 : to_bf16(NAN);
#pragma unroll
    for (int i = 0; i < DPL; ++i) orow[i] = fill;
    if (lane == 0 && p.lse) p.lse[out] = L == 0 ? -INFINITY : NAN;
    return;
  }
  const int ns = (L + kDecodeSplitTokens - 1) / kDecodeSplitTokens;
  float M = lane < ns ? lse0 : kUnset;
  bool bad = lane < ns && lse0 != lse0;
  for (int s = lane + 64; s < ns; s += 64) {
    const float v = lse_s[s];
    bad |= (v != v);
    M = fmaxf(M, v);
  }
  M = wave_max(M);
  bad = __any(bad);
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  // first 64 splits: weights from the loaded log-sum-exps
  const float w0 = lane < ns ? __builtin_amdgcn_exp2f(lse0 - M) : 0.f;
  float W = w0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (c < ns) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w0), c));
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wi, part[c][e], acc[e]);
    }
  }
  for (int c0 = CH; c0 < min(ns, 64); c0 += CH) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int e = 0; e < DPL; ++e)
        part[c][e] = c0 + c < ns ? o_s[(size_t)(c0 + c) * D + e] : 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (c0 + c < ns) {
        const float wi =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w0), c0 + c));
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wi, part[c][e], acc[e]);
      }
    }
  }
  // splits past the first 64 (sequences longer than 64 * 512 tokens)
  for (int s0 = 64; s0 < ns; s0 += 64) {
    const float w = s0 + lane < ns ? __builtin_amdgcn_exp2f(lse_s[s0 + lane] - M) : 0.f;
    W += w;
    const int cnt = min(64, ns - s0);
    for (int i = 0; i < cnt; ++i) {
      const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i));
      const float* src = o_s + (size_t)(s0 + i) * D;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] = fmaf(wi, src[e], acc[e]);
    }
  }
  W = wave_sum(W);
  const float inv = 1.f / W;
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[e] = to_bf16(bad ? NAN : acc[e] * inv);
  if (lane == 0 && p.lse) p.lse[out] = bad ? NAN : (M + __log2f(W)) * kLn2;
}

template <int D>
hipError_t launch_d(const DecParams& p, int N, int layout, bool skip, bool fp8,
                    hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL((decode_fp8_kernel<D, 2>), dim3(p.Hkv, p.n_split, N), dim3(64), 0, stream, p);
  else if (skip && layout == 1)
    hipLaunchKernelGGL((decode_skip_kernel<D>), dim3(p.Hkv, p.n_split, N), dim3(64), 0, stream, p);
  else if (skip)
    hipLaunchKernelGGL((decode_skip_rm_kernel<D>), dim3(p.Hkv, p.n_split, N), dim3(64), 0, stream, p);
  else if (layout == 1)
    hipLaunchKernelGGL((decode_native_kernel<D>), dim3(p.Hkv, p.n_split, N), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<D>), dim3(p.Hkv, p.n_split, N), dim3(64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.Hq, N), dim3(64), 0, stream, p);
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
  // FP8 pools: the K scale multiplies every score, the V scale the output
  p.sl2 = a.scale * (a.fp8 ? a.k_scale : 1.f) * 1.4426950408889634f;
  p.v_scale = a.fp8 ? a.v_scale : 1.f;
  p.G = a.Hq / a.Hkv;
  p.thr = a.skip ? (float)(log((double)a.lambda) * 1.4426950408889634) : 0.f;
  p.skip_map = a.skip_bitmap;
  p.skip_count = a.skip_count;
  if (p.G > 16) return hipErrorInvalidValue;
  if (a.fp8 && a.skip) return hipErrorInvalidValue;
  const bool sk = a.skip != 0, f8 = a.fp8 != 0;
  return a.D == 64 ? launch_d<64>(p, a.N, a.layout, sk, f8, stream)
                   : launch_d<128>(p, a.N, a.layout, sk, f8, stream);
}

}  // namespace attn
