// C-ABI entry points of libattn.so: argument validation, a one-time device
// architecture check, workspace sizing and kernel dispatch.  No entry point
// allocates device memory or synchronises the device.
#include "../../include/attn.h"

#include <math.h>
#include <string.h>

#include <atomic>

#include "attn_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

bool arch_name_ok(const char* name) {
  if (!name) return false;
  // gcnArchName looks like "gfx950" or "gfx950:sramecc+:xnack-"
  return strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

int check_device(int* device = nullptr) {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return ATTN_ERR_NO_DEVICE;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_NO_DEVICE;
  if (dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_HIP;
    st = arch_name_ok(prop.gcnArchName) ? 1 : -1;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  if (device) *device = dev;
  return st == 1 ? ATTN_OK : ATTN_ERR_ARCH;
}

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

int validate_prefill(const void* q, const void* k, const void* v, const void* o, int B, int Hq,
                     int Hkv, int S, int D, int causal, float scale) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1) return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!finite_pos(scale)) return ATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  // element offsets are formed in 64-bit, but each K/V head (S*D) and the
  // grid stay within 32-bit ranges
  if ((long long)S * D > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_ARCH: return "device is not gfx950 (MI355X)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime or launch error";
    case ATTN_ERR_NO_DEVICE: return "no HIP device visible";
    case ATTN_ERR_SCRATCH_LIMIT:
      return "request needs more than the static decode scratch (ATTN_DECODE_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_arch_supported(const char* gcn_arch_name) { return arch_name_ok(gcn_arch_name) ? 1 : 0; }

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int S, int D, int causal, float scale, hipStream_t stream) {
  int st = validate_prefill(q, k, v, o, B, Hq, Hkv, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, 0, 0.f, nullptr, nullptr};
  return hip_status(attn::launch_prefill_bf16(a, stream));
}

int attn_prefill_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                     hipStream_t stream) {
  int st = validate_prefill(q, k, v, o, B, Hq, Hkv, S, D, causal, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::PrefillArgs a{q, k, v, o, lse, B, Hq, Hkv, S, D, causal, scale, 0, 0.f, nullptr, nullptr};
  return hip_status(attn::launch_prefill_f32(a, stream));
}

int attn_prefill_blockskip(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int S, int D, float scale, float lambda,
                           int tile, uint8_t* skip_bitmap, unsigned long long* skipped_tiles,
                           hipStream_t stream) {
  int st = validate_prefill(q, k, v, o, B, Hq, Hkv, S, D, 1, scale);
  if (st != ATTN_OK) return st;
  if (!(lambda > 0.f && lambda < 1.f)) return ATTN_ERR_INVALID_ARG;
  if (tile != 64) return ATTN_ERR_UNSUPPORTED;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::PrefillArgs a{q,  k,     v,      o,           lse,          B, Hq, Hkv, S, D, 1, scale,
                      1, lambda, skip_bitmap, skipped_tiles};
  return hip_status(attn::launch_prefill_bf16(a, stream));
}

size_t attn_decode_workspace_bytes(int num_seqs, int Hq, int D, int max_blocks_per_seq,
                                   int block_size) {
  if (num_seqs < 1 || Hq < 1 || D < 1 || max_blocks_per_seq < 1 || block_size < 1) return 0;
  const size_t ns = (size_t)attn::decode_num_splits(max_blocks_per_seq, block_size);
  return (size_t)num_seqs * Hq * ns * ((size_t)D + 1) * sizeof(float);
}

}  // extern "C"

namespace {

int decode_common(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_table, const int32_t* seq_lens, int block_size,
                  int kv_layout, void* o, float* lse, int num_seqs, int Hq, int Hkv, int D,
                  int num_blocks, int max_blocks_per_seq, float scale, void* workspace,
                  size_t workspace_bytes, int skip, float lambda, uint8_t* skip_bitmap,
                  unsigned long long* skipped_blocks, int fp8, float k_scale, float v_scale,
                  hipStream_t stream, bool static_scratch = false) {
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !o) return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!finite_pos(scale)) return ATTN_ERR_INVALID_ARG;
  if (kv_layout != ATTN_KV_ROWMAJOR && kv_layout != ATTN_KV_MFMA) return ATTN_ERR_INVALID_ARG;
  if (skip && !(lambda > 0.f && lambda < 1.f)) return ATTN_ERR_INVALID_ARG;
  if (fp8 && (!finite_pos(k_scale) || !finite_pos(v_scale))) return ATTN_ERR_INVALID_ARG;
  if (block_size != 16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return ATTN_ERR_UNSUPPORTED;
  const int ns = attn::decode_num_splits(max_blocks_per_seq, block_size);
  if ((long long)ns > 65535 || (long long)Hkv > 65535 || (long long)num_seqs > 65535)
    return ATTN_ERR_UNSUPPORTED;
  const size_t need = attn_decode_workspace_bytes(num_seqs, Hq, D, max_blocks_per_seq, block_size);
  if (static_scratch) {
    if (need > ATTN_DECODE_STATIC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_LIMIT;
  } else {
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 15u) != 0) return ATTN_ERR_WORKSPACE;
  }
  int dev = -1;
  int st = check_device(&dev);
  if (st != ATTN_OK) return st;
  if (static_scratch) {
    // the array's device address on the current GPU, never its host name
    if (attn::decode_static_scratch(dev, &workspace) != hipSuccess) return ATTN_ERR_HIP;
  }
  attn::DecodeArgs a;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.N = num_seqs;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.layout = kv_layout;
  a.scale = scale;
  a.skip = skip;
  a.lambda = lambda;
  a.skip_bitmap = skip_bitmap;
  a.skip_count = skipped_blocks;
  a.fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.n_split = ns;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + (size_t)num_seqs * Hq * ns * D;
  return hip_status(attn::launch_decode_paged(a, stream));
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, int block_size,
                      int kv_layout, void* o, float* lse, int num_seqs, int Hq, int Hkv, int D,
                      int num_blocks, int max_blocks_per_seq, float scale, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, k_pool, v_pool, block_table, seq_lens, block_size, kv_layout, o, lse,
                       num_seqs, Hq, Hkv, D, num_blocks, max_blocks_per_seq, scale, workspace,
                       workspace_bytes, 0, 0.f, nullptr, nullptr, 0, 1.f, 1.f, stream);
}

int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int block_size, int kv_layout, void* o, float* lse, int num_seqs,
                              int Hq, int Hkv, int D, int num_blocks, int max_blocks_per_seq,
                              float scale, hipStream_t stream) {
  return decode_common(q, k_pool, v_pool, block_table, seq_lens, block_size, kv_layout, o, lse,
                       num_seqs, Hq, Hkv, D, num_blocks, max_blocks_per_seq, scale, nullptr, 0, 0,
                       0.f, nullptr, nullptr, 0, 1.f, 1.f, stream, /*static_scratch=*/true);
}

int attn_decode_paged_blockskip(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int block_size, int kv_layout, void* o, float* lse, int num_seqs,
                                int Hq, int Hkv, int D, int num_blocks, int max_blocks_per_seq,
                                float scale, float lambda, uint8_t* skip_bitmap,
                                unsigned long long* skipped_blocks, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return decode_common(q, k_pool, v_pool, block_table, seq_lens, block_size, kv_layout, o, lse,
                       num_seqs, Hq, Hkv, D, num_blocks, max_blocks_per_seq, scale, workspace,
                       workspace_bytes, 1, lambda, skip_bitmap, skipped_blocks, 0, 1.f, 1.f,
                       stream);
}

int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* seq_lens, int block_size,
                          void* o, float* lse, int num_seqs, int Hq, int Hkv, int D,
                          int num_blocks, int max_blocks_per_seq, float scale, float k_scale,
                          float v_scale, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return decode_common(q, k_pool, v_pool, block_table, seq_lens, block_size, ATTN_KV_MFMA, o,
                       lse, num_seqs, Hq, Hkv, D, num_blocks, max_blocks_per_seq, scale, workspace,
                       workspace_bytes, 0, 0.f, nullptr, nullptr, 1, k_scale, v_scale, stream);
}

int attn_prefill_paged(const void* q, const int32_t* cu_seqlens_q, int total_q, int max_seqlen_q,
                       const void* k_pool, const void* v_pool, const int32_t* block_table,
                       const int32_t* seq_lens_k, int block_size, int kv_layout, void* o,
                       float* lse, int num_seqs, int Hq, int Hkv, int D, int num_blocks,
                       int max_blocks_per_seq, float scale, hipStream_t stream) {
  if (!q || !cu_seqlens_q || !k_pool || !v_pool || !block_table || !seq_lens_k || !o)
    return ATTN_ERR_INVALID_ARG;
  if (num_seqs < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      total_q < 1 || max_seqlen_q < 1)
    return ATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID_ARG;
  if (!finite_pos(scale)) return ATTN_ERR_INVALID_ARG;
  if (kv_layout != ATTN_KV_ROWMAJOR && kv_layout != ATTN_KV_MFMA) return ATTN_ERR_INVALID_ARG;
  if (kv_layout != ATTN_KV_ROWMAJOR) return ATTN_ERR_UNSUPPORTED;
  if (block_size != 16) return ATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * 16 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (Hkv > 65535) return ATTN_ERR_UNSUPPORTED;  // pool block bytes stay 32-bit
  int st = check_device();
  if (st != ATTN_OK) return st;
  attn::PagedPrefillArgs a{q,     cu_seqlens_q, k_pool, v_pool, block_table, seq_lens_k,
                           o,     lse,          num_seqs, Hq,    Hkv,         D,
                           num_blocks, max_blocks_per_seq, max_seqlen_q, total_q, scale};
  return hip_status(attn::launch_prefill_paged(a, stream));
}

}  // extern "C"
