// pkv_internal.h -- declarations shared by the C-ABI layer (pkv_api.cpp) and
// the kernels (pkv_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// Everything the split kernel reads, resolved on the host.
struct SplitArgs {
  const uint16_t* query;        // [rows, heads, D] fp16 bits
  const uint8_t* key_cache;     // [pool, B, KVH, D] codes
  const uint8_t* value_cache;   // [pool, B, KVH, VD] codes (SEPARATE)
  const int32_t* block_table;   // [rows, max_blocks_per_row]
  const int32_t* seq_lens;      // [rows]
  const int32_t* candidates;    // [rows, max_candidates] or null
  const int32_t* num_candidates;
  const float* k_scale;         // null for quant NONE
  const float* v_scale;         // LATENT: the K scales
  float* ws_acc;                // [rows, heads, S, VD]
  float* ws_ml;                 // [rows, heads, S, 2]
  int rows, heads, kv_heads, group, head_blocks;
  int qtok;                     // query tokens per row (T >= 1; T > 1: head slots are (token, head))
  int units_row;                // work units per row: kv_heads * head_blocks, or kv_heads / kvp
  int kvp;                      // 4 or 8: that many KV heads per CTA (split_kvp_kernel); else 0
  int block_size, log2_block, max_blocks_per_row, num_pool_blocks, max_candidates;
  int num_splits, min_chunk;
  int target_ctas;              // > 0: live chunk from the total work of all rows
  int grid_ctas;                // 1-D grid of the split kernel
  int static_chunk;             // static mode: positions per split
  int k_quant, v_quant;         // pkv_quant
  int v_scale_stride;           // per-channel V scale row stride (VD, or D for LATENT)
  float score_scale;            // softmax_scale (codes enter the MFMAs at their value)
  float softcap;                // > 0: scores x -> softcap * tanh(x / softcap)
  float inv_softcap;            // 1 / softcap (0 without a cap)
  int window;                   // > 0: sliding window (positions [len - window, len))
  float v_mult;                 // factor applied with the value scale (1)
  // direct output (S = 1): the split kernel writes what the combine would
  // -- O = partial / l with the head sink, and lse -- and no partial
  int direct;
  int out_f32;                  // direct output dtype: FP32 (else FP16)
  void* out;                    // [rows, heads, VD]
  float* lse_out;               // [rows, heads] or null
  const float* head_sink;       // [heads] or null
};

struct CombineArgs {
  const float* ws_acc;
  const float* ws_ml;
  const float* head_sink;       // [heads] or null
  void* out;                    // [rows, heads, VD]
  float* lse_out;               // [rows, heads] or null
  int rows, heads, num_splits;        // rows: query rows (rows x tokens per row)
  int skip_empty;               // read only splits with a nonzero weight
};

// Everything the quantise-on-write kernel reads.  One thread per 8 channels:
// chunks_k = head_size / 8 key chunks, then chunks_v value chunks (0 for
// LATENT) per (token, KV head).
struct WriteArgs {
  const uint16_t* key;          // [tokens, kv_heads, head_size] fp16 bits
  const uint16_t* value;        // [tokens, kv_heads, v_head_size] or null
  const int64_t* slot_mapping;  // [tokens]
  const float* k_scale;
  const float* v_scale;
  uint8_t* key_cache;
  uint8_t* value_cache;
  int64_t n_slots;              // num_pool_blocks * block_size
  int tokens, kv_heads, head_size, v_head_size;
  int chunks_k, chunks_v;
  int k_quant, v_quant;
};

// Kernel variant key.
struct Variant {
  int cache_dtype;  // pkv_dtype
  int head_size, v_head_size;
  int latent;
  int gathered;
  int ext;          // a sliding window or a soft cap is set
  int kvp;          // 4 or 8 KV heads per CTA (dense rows, separate caches); else 0
  int mt;           // several query tokens per row (dense rows, separate caches)
  int vb;           // with kvp: 16-slot head blocks per wave (1, or 2 for 17-32 slots)
};

constexpr int kWaves = 4;          // waves per split-kernel CTA
constexpr int kThreads = 64 * kWaves;
// waves per group and groups per CTA of the latent kernel with one-byte
// codes (with FP16 codes it runs one group of kWaves)
constexpr int kLatentWaves = 4;
constexpr int kLatentGroups = 1;
inline int threads_of(const Variant& v) {
  if (v.kvp > 0) return 64 * v.kvp;  // one wave per KV head
  return (v.latent && v.cache_dtype != PKV_F16) ? 64 * kLatentWaves * kLatentGroups : kThreads;
}
constexpr int kMaxSplits = 64;     // the combine holds one split per lane
constexpr int kMaxBalancedRows = 1024;  // live-balanced chunks up to this many rows
// KV heads of one CTA in the multi-head mode (split_kvp_kernel): four, or
// eight (every head of an eight-KV-head cache record)
constexpr int kKvHeadsPerCta = 4;
constexpr int kKvHeadsPerCtaWide = 8;

// Launchers; return hipSuccess or the launch error.  `supported` reports
// whether a variant was compiled.
bool variant_supported(const Variant& v);
hipError_t launch_split(const Variant& v, const SplitArgs& a, hipStream_t stream);
hipError_t launch_combine(int v_head_size, int out_dtype, const CombineArgs& a, hipStream_t stream);
hipError_t split_occupancy(const Variant& v, int* ctas_per_cu);
hipError_t launch_cache_write(int cache_dtype, const WriteArgs& a, hipStream_t stream);

}  // namespace pkv
