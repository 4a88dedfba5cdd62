// pa_cache_ops.hip - slot write of new tokens and copy-on-write block copy, gfx950.
//
// Both are pure bit copies of whole 16-byte pieces, so they are encoding-agnostic:
//   cache write: a generated token occupies one slot (vLLM-PagedAttention与连续批处理技术
//     拆解, section 3.1). Slot s is row s % 16 of block s / 16; since a block's 16 rows
//     are contiguous, the pool [N, 16, Hkv, d] is also [N * 16, Hkv, d] and slot s
//     starts at byte s * row_bytes (row_bytes = Hkv * d * element bytes).
//   block copy: a shared block is read-only and a writer copies it first (same page,
//     section 3.4); the whole block (16 * row_bytes) is copied for K and for V.
// Entries outside the pool are skipped so that a bad slot or id cannot fault the GPU.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void cache_write_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const uint8_t* __restrict__ k_new,
    const uint8_t* __restrict__ v_new, const int64_t* __restrict__ slots, int32_t num_tokens,
    int32_t row_chunks, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = idx / row_chunks;
  if (t >= num_tokens) return;
  const int64_t c = idx - t * row_chunks;
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;
  const int64_t dst = (s * row_chunks + c) * 16;
  const int64_t src = (t * row_chunks + c) * 16;
  *reinterpret_cast<u32x4*>(k_pool + dst) = *reinterpret_cast<const u32x4*>(k_new + src);
  *reinterpret_cast<u32x4*>(v_pool + dst) = *reinterpret_cast<const u32x4*>(v_new + src);
}

__global__ __launch_bounds__(256) void block_copy_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const int64_t* __restrict__ pairs,
    int32_t num_pairs, int64_t block_chunks, int32_t num_blocks) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t p = idx / block_chunks;
  if (p >= num_pairs) return;
  const int64_t c = idx - p * block_chunks;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t so = (src * block_chunks + c) * 16, d_o = (dst * block_chunks + c) * 16;
  *reinterpret_cast<u32x4*>(k_pool + d_o) = *reinterpret_cast<const u32x4*>(k_pool + so);
  *reinterpret_cast<u32x4*>(v_pool + d_o) = *reinterpret_cast<const u32x4*>(v_pool + so);
}

}  // namespace

hipError_t launch_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t row_bytes, int64_t num_slots, hipStream_t stream) {
  const int32_t row_chunks = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * row_chunks;
  const int64_t blocks = (total + 255) / 256;
  cache_write_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
      static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new), slot_mapping,
      num_tokens, row_chunks, num_slots);
  return hipGetLastError();
}

hipError_t launch_block_copy(void* k_pool, void* v_pool, const int64_t* pairs,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream) {
  const int64_t block_chunks = block_bytes / 16;
  const int64_t total = (int64_t)num_pairs * block_chunks;
  const int64_t blocks = (total + 255) / 256;
  block_copy_kernel<<<dim3((uint32_t)blocks), dim3(256), 0, stream>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), pairs, num_pairs,
      block_chunks, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
