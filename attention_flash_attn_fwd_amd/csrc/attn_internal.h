// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// ---------------------------------------------------------------- launchers
// Each launcher assumes its arguments were validated by the entry point and
// returns the hipError_t of the launch.

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int B, Hq, Hkv, S, D;
  int causal;
  float scale;
  // block skip (ignored unless skip != 0)
  int skip;
  float lambda;
  uint8_t* skip_bitmap;           // may be null
  unsigned long long* skip_count; // may be null
};

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);

// Chunked / variable-length causal prefill over a paged (row-major) cache.
struct PagedPrefillArgs {
  const void* q;              // bf16 [total_q, Hq, D]
  const int32_t* cu_q;        // [N + 1]
  const void* k_pool;         // bf16 [num_blocks, Hkv, 16, D]
  const void* v_pool;
  const int32_t* block_table; // [N, max_blocks]
  const int32_t* seq_lens_k;  // [N]
  void* o;                    // bf16 [total_q, Hq, D]
  float* lse;                 // [total_q, Hq] or null
  int N, Hq, Hkv, D, num_blocks, max_blocks, max_seqlen_q, total_q;
  float scale;
};

hipError_t launch_prefill_paged(const PagedPrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;  // may be null
  int N, Hq, Hkv, D, block_size, num_blocks, max_blocks;
  int layout;  // 0 row-major pools, 1 MFMA-native pools
  float scale;
  // block skip (ignored unless skip != 0; MFMA-native pools only)
  int skip;
  float lambda;
  uint8_t* skip_bitmap;            // may be null
  unsigned long long* skip_count;  // may be null
  // FP8 (E4M3) pools in their own byte order (layout ignored), one scale each
  int fp8;
  float k_scale, v_scale;
  float* ws_o;    // [N, Hq, n_split, D]
  float* ws_lse;  // [N, Hq, n_split]
  int n_split;
};

// Tokens handled by one split-KV workgroup of the decode kernel.
constexpr int kDecodeSplitTokens = 512;

inline int decode_num_splits(int max_blocks, int block_size) {
  long long tokens = (long long)max_blocks * block_size;
  return (int)((tokens + kDecodeSplitTokens - 1) / kDecodeSplitTokens);
}

hipError_t launch_decode_paged(const DecodeArgs& a, hipStream_t stream);

// Device address of the library's static decode scratch
// (ATTN_DECODE_STATIC_SCRATCH_BYTES) on `device`, which must be the current
// device.  Resolved with hipGetSymbolAddress on the first call per device and
// kept; later calls make no HIP call.
hipError_t decode_static_scratch(int device, void** addr);

}  // namespace attn
