/*
 * attn.h - exact attention computed IO-aware on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Every entry point enqueues work asynchronously on the
 * given HIP stream and returns an attn_status code; it never synchronises the
 * device.  All tensor pointers are DEVICE pointers owned by the caller; the
 * library allocates no device memory and keeps no state between calls apart
 * from a one-time check of the device architecture and, for
 * attn_decode_paged_noalloc, a static scratch array per GPU (part of the
 * library's code object) and its device address.  Arguments are validated
 * on the host before any HIP call; a call that returns an error has enqueued
 * nothing.  Values inside device buffers (sequence lengths, block-table
 * entries) cannot be checked on the host: see attn_decode_paged for how the
 * kernels treat bad ones.
 *
 * Layouts (row-major, contiguous):
 *   prefill  Q, O : [B, Hq,  S, D]     K, V : [B, Hkv, S, D]
 *            LSE  : float32 [B, Hq, S], natural logarithm
 *   decode   q, o : [N, Hq, D]         lse  : float32 [N, Hq]
 *            k_pool, v_pool : see attn_kv_layout
 *            block_table    : int32 [N, max_blocks_per_seq]
 *            seq_lens       : int32 [N]
 *   bf16 tensors hold IEEE bfloat16 bit patterns (uint16_t).
 *
 * Grouped-query attention: Hq must be a multiple of Hkv and query head h uses
 * key/value head h / (Hq / Hkv), i.e. each K/V head serves Hq/Hkv consecutive
 * query heads ("TensorRT对Grouped Query Attention的支持进展", sub-sections
 * 技术演进背景 and 图优化与算子融合: query heads split into groups sharing one
 * K/V head; the repeat_kv plugin repeats each K/V head for its group).
 * Hkv == Hq is multi-head attention, Hkv == 1 multi-query attention.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layouts of the paged K/V pools.  Both keep each (block, head) as one
 * contiguous run of block_size * D elements; only the order inside the run
 * differs.
 *   ATTN_KV_ROWMAJOR: k_pool, v_pool [num_blocks, Hkv, block_size, D]
 *   ATTN_KV_MFMA:     k_pool [num_blocks, Hkv, D/8, block_size, 8]  (8-element
 *                     chunks of each token row, chunk-major)
 *                     v_pool [num_blocks, Hkv, D, block_size]       (V transposed
 *                     within the block)
 * The MFMA layout lets every matrix-core operand be one coalesced load
 * straight from HBM and is the faster one. */
typedef enum { ATTN_KV_ROWMAJOR = 0, ATTN_KV_MFMA = 1 } attn_kv_layout;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, Hq % Hkv != 0, ... */
  ATTN_ERR_UNSUPPORTED = -2, /* well-formed but not built: D not in {64,128}, ...   */
  ATTN_ERR_ARCH = -3,        /* current device is not gfx950                         */
  ATTN_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required           */
  ATTN_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed           */
  ATTN_ERR_NO_DEVICE = -6,   /* no HIP device is visible                             */
  ATTN_ERR_SCRATCH_LIMIT = -7 /* request needs more than the static scratch of
                                 attn_decode_paged_noalloc                            */
} attn_status;

/* Size of the static device scratch array that attn_decode_paged_noalloc
 * uses in place of a caller workspace (one copy per GPU, held until the
 * process ends). */
#define ATTN_DECODE_STATIC_SCRATCH_BYTES (16u << 20)

/* Static, human-readable text for a status code (never NULL).  Plumbing of
 * this interface: no passage of the source pages defines it. */
const char* attn_status_string(int status);

/* 1 if a device whose gcnArchName is `gcn_arch_name` (e.g. "gfx950" or
 * "gfx950:sramecc+:xnack-") can run this library, else 0.  Pure function: it
 * makes no HIP call.  The entry points apply the same test to the current
 * device on first use and return ATTN_ERR_ARCH when it fails. */
int attn_arch_supported(const char* gcn_arch_name);

/*
 * attn_prefill - exact causal or non-causal attention of S queries over the
 * same S keys, bf16 in, bf16 out, fp32 accumulation.
 *
 * Computes, for every batch b, query head h (K/V head g = h / (Hq/Hkv)) and
 * query row i:  s_ij = scale * <q_i, k_j>;  O_i = sum_j softmax_j(s_i.) v_j;
 * LSE_i = ln sum_j exp(s_ij), over keys j <= i when causal != 0, else all j.
 * This is the exact attention that FlashAttention computes IO-aware
 * ("flash-attention与TensorRT-LLM集成", FlashAttention working principle:
 * Q, K, V are split into blocks processed on chip, so the S x S score matrix
 * is never stored and memory stays linear in S).  The kernel tiles Q.K^T,
 * keeps a running row maximum and sum (online softmax) and accumulates P.V in
 * one pass; K/V tiles are staged once in LDS and shared by the query heads of
 * a GQA group.
 *
 *   q, k, v : bf16 device pointers, layouts above;  o : bf16 [B,Hq,S,D] (out)
 *   lse     : float32 [B,Hq,S] (out), may be NULL when not wanted
 *   B, Hq, Hkv, S >= 1, Hq % Hkv == 0, D in {64, 128}
 *   causal  : 0 or 1 (key j visible to query i iff j <= i)
 *   scale   : positive finite score scale, typically 1/sqrt(D)
 * Errors: ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ARCH,
 * ATTN_ERR_NO_DEVICE, ATTN_ERR_HIP.  O and LSE are untouched on error.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                 hipStream_t stream);

/*
 * attn_prefill_f32 - as attn_prefill with float32 Q, K, V and O and true fp32
 * products and sums throughout (no bf16/tf32 rounding anywhere).  The same
 * operation as attn_prefill (same passage); the pages name no number type,
 * and this entry point serves the fp32 workload.
 */
int attn_prefill_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                     hipStream_t stream);

/*
 * attn_prefill_blockskip - causal bf16 prefill that skips negligible tiles
 * ("高效部署稀疏注意力加速方案：BLASST方法详解与实践指南", 架构与组件: from the
 * running maximum of the blockwise online softmax and a threshold lambda,
 * decide whether a block matters; for blocks that do not, skip the softmax
 * exponentials, the V load and the matrix product).
 *
 * Key tiles of `tile` keys are visited in ascending order for each query tile
 * of `tile` rows and each query head.  With m_r the running maximum of row r's
 * scaled scores over the tiles already visited and tm_r the row's maximum over
 * its visible keys in the current tile, row r is negligible iff tm_r = -inf or
 * (m_r is defined and tm_r - m_r < ln(lambda)); the tile is skipped (no exp,
 * no P.V, no update of the row statistics) iff all of its rows are negligible.
 * O and LSE are then exact attention over the keys of the tiles not skipped.
 * The V rows of key tile kt are not read from memory when every query tile
 * processed together with it (up to four query heads of the K/V group, 64
 * rows each) skips kt.
 *
 *   lambda        : 0 < lambda < 1
 *   tile          : must be 64
 *   skip_bitmap   : optional uint8 [B, Hq, nT, nT], nT = ceil(S/64); entry
 *                   [b,h,qt,kt] for kt <= qt is set to 1 (skipped) or 0; entries
 *                   with kt > qt are not written.  May be NULL.
 *   skipped_tiles : optional device uint64 counter; the number of skipped
 *                   (b, h, qt, kt) tiles is ADDED to it (the caller zeroes it).
 *                   May be NULL.
 * Other arguments and errors as attn_prefill (causal is implied).
 */
int attn_prefill_blockskip(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int S, int D, float scale,
                           float lambda, int tile, uint8_t* skip_bitmap,
                           unsigned long long* skipped_tiles, hipStream_t stream);

/*
 * attn_decode_workspace_bytes - device workspace attn_decode_paged needs for
 * the given sizes (0 for invalid sizes).  Holds one partial output and one
 * partial log-sum-exp per (sequence, query head, KV split).  Plumbing of the
 * split-KV decode: no passage of the source pages defines it.
 */
size_t attn_decode_workspace_bytes(int num_seqs, int Hq, int D, int max_blocks_per_seq,
                                   int block_size);

/*
 * attn_decode_paged - one new query token per sequence attending to that
 * sequence's cached keys/values, gathered through a block table
 * ("LLM推理优化技术综述：KVCache、PageAttention、FlashAttention、MQA、GQA",
 * PageAttention part: the KV cache is cut into fixed-size blocks and a block
 * table maps each sequence's contiguous logical blocks to non-contiguous
 * physical blocks; "TensorRT-LLM：大模型推理加速的工业级引擎", PagedAttention
 * section).  Cached token t of sequence n is slot t % block_size of physical
 * block block_table[n][t / block_size]; the query attends to all
 * L = seq_lens[n] cached tokens (no mask).
 *
 * The key range of each sequence is split into chunks processed by separate
 * workgroups (split-KV); partial outputs and log-sum-exps go to `workspace`
 * and a second kernel merges them: lse = ln sum_s exp(lse_s),
 * O = sum_s exp(lse_s - lse) O_s.
 *
 *   q            : bf16 [N, Hq, D];  o : bf16 [N, Hq, D] (out)
 *   lse          : float32 [N, Hq] (out) or NULL
 *   k_pool/v_pool: bf16 pools in the layout kv_layout names (attn_kv_layout)
 *   kv_layout    : ATTN_KV_ROWMAJOR or ATTN_KV_MFMA
 *   block_table  : int32 [N, max_blocks_per_seq]; unused entries are ignored.
 *                  Entries of different sequences may name the same physical
 *                  block (prompt blocks shared copy-on-write between the
 *                  samples of one prompt, same page, PageAttention part): the
 *                  pools are only read.
 *   seq_lens     : int32 [N]
 *   block_size   : must be 16;  D in {64, 128};  Hq % Hkv == 0, Hq/Hkv <= 16
 *   workspace    : device buffer of at least
 *                  attn_decode_workspace_bytes(N, Hq, D, max_blocks_per_seq, 16) bytes
 * Device-side values: a sequence with seq_lens[n] == 0 gets O = 0 and
 * LSE = -inf.  A sequence whose length exceeds max_blocks_per_seq*block_size,
 * is negative, or whose table holds an entry outside [0, num_blocks) for a
 * block it uses, gets NaN in O and LSE for every head (no out-of-range memory
 * is read).  Errors: ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_ARCH, ATTN_ERR_NO_DEVICE, ATTN_ERR_HIP.
 */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, int block_size,
                      int kv_layout, void* o, float* lse, int num_seqs, int Hq, int Hkv, int D,
                      int num_blocks, int max_blocks_per_seq, float scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_paged_noalloc - attn_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and result as
 * attn_decode_paged (the same kernels run), without the workspace: the
 * split-KV partial results go to a static device array inside the library,
 * ATTN_DECODE_STATIC_SCRATCH_BYTES per GPU, whose address is looked up once
 * per device on the first call made with that device current.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *   A request whose attn_decode_workspace_bytes(num_seqs, Hq, D,
 *   max_blocks_per_seq, 16) exceeds ATTN_DECODE_STATIC_SCRATCH_BYTES is
 *   rejected with ATTN_ERR_SCRATCH_LIMIT before anything is enqueued (e.g.
 *   64 sequences x 32 query heads x D = 128 fit with up to 7680 tokens,
 *   480 blocks of 16, per table row).
 * Every call on one GPU shares that GPU's array, and each call overwrites
 * the part it uses before reading it: calls that can overlap on one GPU
 * (different streams without ordering between them) race on it and must be
 * serialised by the caller.  Other errors as attn_decode_paged, except that
 * ATTN_ERR_WORKSPACE does not occur.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int block_size, int kv_layout, void* o, float* lse, int num_seqs,
                              int Hq, int Hkv, int D, int num_blocks, int max_blocks_per_seq,
                              float scale, hipStream_t stream);

/* Paged decode with block skipping ("高效部署稀疏注意力加速方案：BLASST方法详解与
 * 实践指南", 架构与组件: a running maximum from the blockwise online softmax and
 * a threshold lambda decide which blocks matter; the others lose their exp,
 * their V load and their matrix product).  Arguments as attn_decode_paged
 * (either pool layout), plus:
 *   lambda        : threshold, 0 < lambda < 1
 *   skip_bitmap   : uint8 [N, Hkv, max_blocks_per_seq] or NULL; entry
 *                   (n, g, j) is set to 1 if logical block j of sequence n
 *                   was skipped for K/V head g, 0 if kept; entries past the
 *                   sequence are not written
 *   skipped_blocks: device counter or NULL, incremented by the number of
 *                   skipped (sequence, K/V head, block) triples; the caller
 *                   zeroes it
 * Rule: each sequence's tokens are cut into the same 512-token splits as
 * the split-KV decode; inside a split the blocks are taken in order, and
 * block j is skipped when for every query head h of the K/V group its
 * maximum scaled score minus the maximum over the split's earlier blocks is
 * below ln(lambda).  A split's first block is always kept.  O and LSE are
 * the attention over the kept blocks' tokens. */
int attn_decode_paged_blockskip(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int kv_layout, void* o, float* lse, int num_seqs,
                                int Hq, int Hkv, int D, int num_blocks, int max_blocks_per_seq,
                                float scale, float lambda, uint8_t* skip_bitmap,
                                unsigned long long* skipped_blocks, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Paged decode over an FP8 KV cache.  The TensorRT-LLM page lists FP8 among
 * its low-precision formats ("TensorRT-LLM：大模型推理加速的工业级引擎",
 * 六大核心优化技术 / 量化; its 深入版解读 names the E4M3/E5M2 encodings) and the
 * integration page enables FP8 with the KV cache ("flash-attention与TensorRT-
 * LLM集成", 案例研究：Mistral-7B部署); neither gives a scale convention, so this entry
 * point takes E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities, S.1111.111 is NaN, largest finite 448) with ONE fp32 scale per
 * pool: cached K value = k_scale * code value, V value = v_scale * code value.
 * The attention is then exactly that of attn_decode_paged on those values.
 * Arguments as attn_decode_paged (no kv_layout), except:
 *   k_pool, v_pool : uint8 codes, [num_blocks, Hkv, 16 * D], one run of 16 * D
 *                    bytes per (block, K/V head), D % 64 == 0, in this order
 *                    (token t in [0, 16), dim d, c = d / 16):
 *                      K code at (c / 4) * 1024 + ((c % 4) * 16 + t) * 16 + d % 16
 *                      V code at (c / 4) * 1024 + ((t / 4) * 16 + d % 16) * 16
 *                                + (c % 4) * 4 + t % 4
 *   k_scale, v_scale: finite and > 0 (ATTN_ERR_INVALID_ARG otherwise)
 * q, o stay bf16 and lse fp32.  Slots past a sequence's end may hold any
 * byte, NaN codes included; they are never used.  Same device-side rules,
 * workspace and errors as attn_decode_paged. */
int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* seq_lens, int block_size,
                          void* o, float* lse, int num_seqs, int Hq, int Hkv, int D,
                          int num_blocks, int max_blocks_per_seq, float scale, float k_scale,
                          float v_scale, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Chunked / variable-length causal prefill over the paged KV cache (the
 * prefill-with-KV-cache case of "flash-attention与TensorRT-LLM集成" and the
 * block table of "LLM推理优化技术综述", PageAttention part).  Sequence n
 * has Sk = seq_lens_k[n] tokens whose K/V are already in the pools (earlier
 * context and the new chunk); its Sq = cu_seqlens_q[n+1] - cu_seqlens_q[n]
 * queries are its last Sq positions: query i sees the keys
 * j <= Sk - Sq + i (causal, bottom-right aligned).
 *   q, o          : bf16 [total_q, Hq, D], packed sequence after sequence
 *   cu_seqlens_q  : int32 [num_seqs + 1], cu[0] = 0, cu[num_seqs] = total_q
 *   max_seqlen_q  : an upper bound on every Sq (sizes the grid)
 *   lse           : float32 [total_q, Hq] (natural log) or NULL
 *   k_pool/v_pool : bf16, kv_layout must be ATTN_KV_ROWMAJOR
 *                   ([num_blocks, Hkv, 16, D]; ATTN_ERR_UNSUPPORTED otherwise)
 *   block_table   : int32 [num_seqs, max_blocks_per_seq]
 * Hkv above 65535 gives ATTN_ERR_UNSUPPORTED, as in the decode.
 * Device-side values are checked by the kernel before anything is read
 * through them.  A sequence n with cu_seqlens_q[n] < 0, cu_seqlens_q[n+1] >
 * total_q, cu_seqlens_q[n+1] < cu_seqlens_q[n], Sq > max_seqlen_q, Sq > Sk,
 * Sk < 0, Sk > 16 * max_blocks_per_seq, or a table entry outside
 * [0, num_blocks) among the ceil(Sk/16) blocks it uses gets NaN in O and LSE
 * for its rows [max(cu[n], 0), min(cu[n+1], total_q)) (none if that range is
 * empty); no other row is written and no memory outside q, the pools, the
 * table and the offsets is read. */
int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q, int total_q, int max_seqlen_q,
                       const void* k_pool, const void* v_pool, const int32_t* block_table,
                       const int32_t* seq_lens_k, int block_size, int kv_layout, void* o,
                       float* lse, int num_seqs, int Hq, int Hkv, int D, int num_blocks,
                       int max_blocks_per_seq, float scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
