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
//
// The slot write into an fp8 cache quantises each new value instead of copying bits
// (the fp8 E4M3 KV cache of the same page, section 五): y = fp32(x) * inv_scale (one
// binary32 multiply, inv_scale = fp32(1 / scale) from the host), then the nearest OCP
// E4M3FN value with ties to even. y is clamped to +-448 first, so values past the
// largest finite one saturate whatever the conversion does with them, and NaN is
// encoded as 0x7F explicitly.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_attention.h"
#include "pa_launch.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

// Two binary32 values -> two E4M3FN codes (a in the low byte).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  const float ac = a != a ? 0.0f : fminf(fmaxf(a, -448.0f), 448.0f);
  const float bc = b != b ? 0.0f : fminf(fmaxf(b, -448.0f), 448.0f);
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, ac, bc, 1.0f, false);
  uint32_t w = __builtin_bit_cast(uint32_t, r) & 0xffffu;
  if (a != a) w = (w & 0xff00u) | 0x7fu;
  if (b != b) w = (w & 0x00ffu) | 0x7f00u;
  return w;
}

// 8 source values (16 bytes of fp16/bf16, 32 of fp32) at element offset e -> 8 codes
template <int SRC>
__device__ __forceinline__ u32x2 quant8(const uint8_t* src, int64_t e, float inv) {
  float x[8];
  if constexpr (SRC == PA_F32) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(src + e * 4);
    const u32x4 b = *reinterpret_cast<const u32x4*>(src + e * 4 + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(a[i]);
      x[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(src + e * 2);
    if constexpr (SRC == PA_F16) {
      const f16x8 h = __builtin_bit_cast(f16x8, a);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(a[i] << 16);
        x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
      }
    }
  }
  u32x2 o;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    o[i] = e4m3_pair(x[4 * i] * inv, x[4 * i + 1] * inv) |
           e4m3_pair(x[4 * i + 2] * inv, x[4 * i + 3] * inv) << 16;
  return o;
}

template <int SRC>
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, const uint8_t* __restrict__ k_new,
    const uint8_t* __restrict__ v_new, const int64_t* __restrict__ slots, int32_t num_tokens,
    int32_t row_octs, int64_t num_slots, float k_inv, float v_inv,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales, int32_t head_octs) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = idx / row_octs;
  if (t >= num_tokens) return;
  const int64_t c = idx - t * row_octs;              // 8-element piece of the row
  const int64_t s = slots[t];
  if (s < 0 || s >= num_slots) return;
  if (k_scales) {
    // per-head scales: the piece lies in kv head c / head_octs; one binary32 reciprocal,
    // rounded to nearest like the host's for a per-tensor scale
    const int64_t g = c / head_octs;
    k_inv = __fdiv_rn(1.0f, k_scales[g]);
    v_inv = __fdiv_rn(1.0f, v_scales[g]);
  }
  const int64_t e = (t * row_octs + c) * 8;          // source element
  const int64_t dst = (s * row_octs + c) * 8;        // pool byte (one byte per element)
  *reinterpret_cast<u32x2*>(k_pool + dst) = quant8<SRC>(k_new, e, k_inv);
  *reinterpret_cast<u32x2*>(v_pool + dst) = quant8<SRC>(v_new, e, v_inv);
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

hipError_t launch_cache_write_fp8(void* k_pool, void* v_pool, const void* k_new,
                                  const void* v_new, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t row_elems, int64_t num_slots,
                                  int32_t src_dtype, float k_inv, float v_inv,
                                  const float* k_head_scales, const float* v_head_scales,
                                  int32_t head_dim, hipStream_t stream) {
  const int32_t row_octs = row_elems / 8;
  const int32_t head_octs = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * row_octs;
  const dim3 grid((uint32_t)((total + 255) / 256)), block(256);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  auto* kn = static_cast<const uint8_t*>(k_new);
  auto* vn = static_cast<const uint8_t*>(v_new);
  switch (src_dtype) {
    case PA_F32:
      cache_write_fp8_kernel<PA_F32><<<grid, block, 0, stream>>>(
          kp, vp, kn, vn, slot_mapping, num_tokens, row_octs, num_slots, k_inv, v_inv,
          k_head_scales, v_head_scales, head_octs);
      break;
    case PA_F16:
      cache_write_fp8_kernel<PA_F16><<<grid, block, 0, stream>>>(
          kp, vp, kn, vn, slot_mapping, num_tokens, row_octs, num_slots, k_inv, v_inv,
          k_head_scales, v_head_scales, head_octs);
      break;
    case PA_BF16:
      cache_write_fp8_kernel<PA_BF16><<<grid, block, 0, stream>>>(
          kp, vp, kn, vn, slot_mapping, num_tokens, row_octs, num_slots, k_inv, v_inv,
          k_head_scales, v_head_scales, head_octs);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Whole blocks from one pool to another, K and V; either pool may be pinned host memory
// (swap-out and swap-in of preempted sequences). Workgroup w copies 4 KB pieces of pair
// w / gx (so the pair is read once per wave, as a uniform load), 16 bytes per thread.
__global__ __launch_bounds__(256) void block_swap_kernel(
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, int32_t dst_blocks,
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v, int32_t src_blocks,
    const int64_t* __restrict__ pairs, int64_t block_chunks, int32_t gx) {
  const int p = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / (uint32_t)gx));
  const int part = (int)blockIdx.x - p * gx;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  for (int64_t c = (int64_t)part * 256 + threadIdx.x; c < block_chunks; c += (int64_t)gx * 256) {
    const int64_t so = (src * block_chunks + c) * 16, d_o = (dst * block_chunks + c) * 16;
    const u32x4 k = *reinterpret_cast<const u32x4*>(src_k + so);
    const u32x4 v = *reinterpret_cast<const u32x4*>(src_v + so);
    *reinterpret_cast<u32x4*>(dst_k + d_o) = k;
    *reinterpret_cast<u32x4*>(dst_v + d_o) = v;
  }
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

hipError_t launch_block_swap(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k,
                             const void* src_v, int32_t src_blocks, const int64_t* pairs,
                             int32_t num_pairs, int64_t block_bytes, hipStream_t stream) {
  const int64_t block_chunks = block_bytes / 16;
  const int64_t per_pair = (block_chunks + 255) / 256;
  const int32_t gx = (int32_t)(per_pair < 64 ? per_pair : 64);
  block_swap_kernel<<<dim3((uint32_t)((int64_t)num_pairs * gx)), dim3(256), 0, stream>>>(
      static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), dst_blocks,
      static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v), src_blocks, pairs,
      block_chunks, gx);
  return hipGetLastError();
}

}  // namespace pa
