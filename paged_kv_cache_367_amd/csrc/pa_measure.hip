// pa_measure.hip - a streaming read of device memory, gfx950: the read-only bandwidth
// reference that a kernel which only reads HBM (as the decode does) can be set against.
//
// Workgroup w reads its own contiguous slab of the buffer, 32 KB per step (eight 16-byte
// loads in flight per thread, streaming (nt) loads through a buffer descriptor that ends
// with the buffer, so the last slab needs no bounds checks). The words are folded with
// XOR and a thread stores only if its fold equals a fixed pattern, so the loads cannot
// be dropped and the kernel writes (almost) nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kReadUnroll = 8;
constexpr int kReadThreads = 256;
constexpr uint32_t kReadStep = kReadUnroll * kReadThreads * 16;   // bytes per workgroup step

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint8_t* src,
                                                                   uint64_t bytes,
                                                                   uint64_t slab,
                                                                   uint32_t* sink) {
  const uint64_t beg = (uint64_t)blockIdx.x * slab;
  if (beg >= bytes) return;
  const uint32_t len = (uint32_t)(bytes - beg < slab ? bytes - beg : slab);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src + beg, len);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (uint32_t off = 0; off < len; off += kReadStep) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      v[u] = buf_load16<kStream>(r, off + (uint32_t)(u * kReadThreads + threadIdx.x) * 16u);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

// `workgroups` workgroups, each reading a slab of ceil(bytes / workgroups) rounded up to
// whole steps; slabs stay below 2^32 bytes (the descriptor's size field).
hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream) {
  uint64_t slab = (bytes + workgroups - 1) / workgroups;
  slab = (slab + kReadStep - 1) / kReadStep * kReadStep;
  if (slab >= ((uint64_t)1 << 32)) return hipErrorInvalidValue;
  const uint64_t grid = (bytes + slab - 1) / slab;
  stream_read_kernel<<<dim3((unsigned)grid), dim3(kReadThreads), 0, stream>>>(
      static_cast<const uint8_t*>(src), bytes, slab, sink);
  return hipGetLastError();
}

}  // namespace pa
