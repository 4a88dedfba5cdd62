// pa_launch.h - internal launch interface between the C ABI (pa_api.cpp) and the HIP
// kernels (pa_decode.hip, pa_cache_ops.hip). Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;      // tokens per KV block (the only supported size)
constexpr int kDecodeWaves = 4;       // waves per decode workgroup
constexpr int kMaxPartitionTokens = 4096;
constexpr int kDefaultPartitionTokens = 512;

// Arguments of the split-KV decode kernel. One workgroup handles one
// (partition, kv head, sequence) triple.
struct DecodeArgs {
  void* out;                    // [B, Hq, d] out dtype
  const void* q;                // [B, Hq, d] q dtype
  const void* k_pool;           // [N, 16, Hkv, d]
  const void* v_pool;
  const int32_t* block_tables;  // [B, maxb]
  const int32_t* context_lens;  // [B]
  float* ws_acc;                // [B, Hq, max_parts, d]   (only when max_parts > 1)
  float* ws_ml;                 // [B, Hq, max_parts, 2]   (m in log2 units, l)
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t part_blocks;          // blocks per partition
  int32_t max_parts;            // partitions covering max_context_len
  float qk_scale_log2;          // scale * k_scale * log2(e)
  float v_scale;
};

// Arguments of the cross-partition merge kernel. One wave per (sequence, query head).
struct MergeArgs {
  void* out;
  const int32_t* context_lens;
  const float* ws_acc;
  const float* ws_ml;
  int32_t num_q_heads;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t part_blocks;
  int32_t max_parts;
  float v_scale;
};

hipError_t launch_decode(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                         const DecodeArgs& args, int batch, hipStream_t stream);
hipError_t launch_merge(int out_dtype, int head_dim, const MergeArgs& args, int batch,
                        hipStream_t stream);

hipError_t launch_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t row_bytes, int64_t num_slots, hipStream_t stream);
hipError_t launch_block_copy(void* k_pool, void* v_pool, const int64_t* pairs,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream);

}  // namespace pa
