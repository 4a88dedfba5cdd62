// pa_device.h - device helpers shared by the HIP kernels (gfx950): vector types, storage
// encodings, raw buffer loads, cross-lane moves and output conversion. Internal; not
// part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_attention.h"

namespace pa {
namespace {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x1 __attribute__((ext_vector_type(1)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int T> struct Enc;
template <> struct Enc<PA_F32> { static constexpr int bytes = 4; };
template <> struct Enc<PA_F16> { static constexpr int bytes = 2; };
template <> struct Enc<PA_BF16> { static constexpr int bytes = 2; };
template <> struct Enc<PA_FP8_E4M3> { static constexpr int bytes = 1; };

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane moves inside 16-lane rows.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// A value the whole wave agrees on (an LDS word read at a uniform address), marked as
// such so that what is derived from it stays in scalar registers; without this the
// compiler wraps every load whose descriptor depends on it in a per-lane loop.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Make LDS writes of this wave visible to its own later LDS reads from other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), other counters untouched
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer loads: the block base lives in a scalar descriptor, each lane adds a
// constant 32-bit offset. Offsets at or beyond `bytes` read as zero without touching
// memory, which gives past-the-end prefetches for free (bytes = 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Cache policy of a load: kCached, or kStream (the nt bit: data read once, which the caches
// should not keep; streaming reads reach more HBM bandwidth with it).
constexpr int kCached = 0, kStream = 2;
template <int POL = kCached>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, POL));
}
template <int POL = kCached>
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, POL));
}

// fp32 -> bf16, round to nearest even (the hardware conversion of CDNA4)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int OT>
__device__ __forceinline__ void store_out(void* out, size_t idx, float x) {
  if constexpr (OT == PA_F32) {
    static_cast<float*>(out)[idx] = x;
  } else if constexpr (OT == PA_F16) {
    static_cast<_Float16*>(out)[idx] = (_Float16)x;
  } else {
    static_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(x);
  }
}

// Max and sum over the four row groups of a column: lanes l, l ^ 16, l ^ 32, l ^ 48.
// v_permlane16_swap / v_permlane32_swap exchange rows 0<->1, 2<->3 and the two halves,
// so with both operands equal, the pair returned holds each lane's value and its
// partner's, in some order.
__device__ __forceinline__ float xrow_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  x = a > b ? a : b;
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  const float c = __uint_as_float(r2[0]), d = __uint_as_float(r2[1]);
  return c > d ? c : d;
}
__device__ __forceinline__ float xrow_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}

template <int POL = kCached>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, POL);
}

// Loads of 16, 8 or 4 bytes per lane through a buffer descriptor, with cache policy POL.
template <int BYTES> struct VChunk;
template <> struct VChunk<16> {
  using type = u32x4;
  template <int POL = kCached>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return buf_load16<POL>(r, o);
  }
};
template <> struct VChunk<8> {
  using type = u32x2;
  template <int POL = kCached>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return buf_load8<POL>(r, o);
  }
};
template <> struct VChunk<4> {
  using type = u32x1;
  template <int POL = kCached>
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    u32x1 v;
    v[0] = buf_load4<POL>(r, o);
    return v;
  }
};

}  // namespace
}  // namespace pa
