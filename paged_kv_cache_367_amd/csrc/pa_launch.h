// pa_launch.h - internal launch interface between the C ABI (pa_api.cpp) and the HIP
// kernels (pa_decode.hip, pa_prefill.hip, pa_cache_ops.hip). Not installed; not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;      // tokens per KV block (the only supported size)
constexpr int kMaxGroupWaves = 8;     // waves per decode workgroup (= kv heads per head group)
constexpr int kMaxDeviceCUs = 256;    // the grid uses at most this many CUs (an MI355X has 256)
constexpr int kWavesPerCU = 8;        // decode registers are sized for 2 waves per SIMD
constexpr int kMaxPartitionTokens = 1 << 20;
constexpr int kMaxBatch = 4096;       // lengths and prefix sums of the batch sit in LDS

// Work split of one decode call. A unit is one 16-token block of one sequence for one
// head group (kv heads hg*NW .. hg*NW + NW - 1). Units are numbered sequence-major, then
// head group, then logical block, so each (sequence, head group) is a contiguous segment
// of nb = ceil(L / 16) units. There are T = (Hkv / NW) * sum_b nb units, cut into chunks;
// a workgroup of NW waves (one per kv head of the group) walks its chunks unit by unit.
// A segment cut by a chunk boundary leaves one (m, l, acc) record per piece, which
// merge kernels combine; a segment inside one chunk is written out directly.
//
// Chunks of [0, T), numbered in unit order: W equal static chunks, chunk c =
// [T*c/W, T*(c+1)/W) (a chunk may be empty when T < W), workgroup r of the W0 in the grid
// taking the contiguous run r*m .. r*m + m - 1. Default split: m = 1 (W = W0). With a
// fixed partition of P units: m = ceil(T / (W0 P)), the smallest number of chunks per
// workgroup for which no chunk holds more than P units.
struct ChunkGeom {
  int64_t T;
  int W, per_wg;      // chunks, chunks per workgroup (m)
  bool fixed;
  int q, r, wshift;   // T = q * W + r; wshift = log2(W) when W is a power of two, else -1
};
constexpr int64_t kMaxChunks = 16384;

// T < 2^31 (the host checks unit counts) and W <= kMaxChunks, so static chunk bounds need
// only 32-bit products (r * c < W^2 < 2^28), and a shift when W is a power of two.
__host__ __device__ inline ChunkGeom chunk_geometry(int64_t T, int W0, int fixed_units) {
  ChunkGeom g;
  g.T = T;
  g.fixed = fixed_units > 0;
  const int64_t per = (int64_t)W0 * (fixed_units > 0 ? fixed_units : 1);
  g.per_wg = g.fixed && T > per ? (int)((T + per - 1) / per) : 1;
  g.W = W0 * g.per_wg;
  const int W = g.W;
  g.wshift = (W & (W - 1)) == 0 ? __builtin_ctz((unsigned)W) : -1;
  const int Ti = (int)T;
  g.q = g.wshift >= 0 ? Ti >> g.wshift : Ti / W;
  g.r = Ti - g.q * W;
  return g;
}
// floor(T * c / W) for 0 <= c <= W
__host__ __device__ inline int64_t static_bound(const ChunkGeom& g, int c) {
  const int rc = g.r * c;
  return (int64_t)g.q * c + (g.wshift >= 0 ? rc >> g.wshift : rc / g.W);
}
__host__ __device__ inline int64_t chunk_begin(const ChunkGeom& g, int c) {
  return static_bound(g, c);
}
__host__ __device__ inline int64_t chunk_end(const ChunkGeom& g, int c) {
  return static_bound(g, c + 1);
}
// chunk holding unit u (0 <= u < T): the last chunk starting at or before u, i.e.
// floor(((u + 1) W - 1) / T). In double precision, which is exact here and far shorter
// than a 64-bit integer division on the GPU: the numerator is below 2^45 (u < 2^31,
// W <= kMaxChunks) and the quotient below 2^14, so a quotient that is not an integer lies
// at least 1/T, a relative 2^-45, below the next one, and rounding to 53 bits cannot
// carry it there.
__host__ __device__ inline int chunk_of(const ChunkGeom& g, int64_t u) {
  return (int)(((double)(u + 1) * (double)g.W - 1.0) / (double)g.T);
}

struct DecodeArgs {
  void* out;                    // [B, Hq, d] out dtype
  const void* q;                // [B, Hq, d] q dtype
  const void* k_pool;           // [N, 16, Hkv, d]
  const void* v_pool;
  const int32_t* block_tables;  // [B, maxb]
  const int32_t* context_lens;  // [B]
  float* rec_acc;               // [chunks, 2, NW, G, d]  unnormalised partial outputs
  float* rec_ml;                // [chunks, 2, NW, G, 2]  (running max m in log2 units, sum l)
  int32_t* prefix;              // [B + 1] blocks before each sequence (workgroup 0 writes)
  int32_t* chunk_hdr;           // [chunks][4] default split: the cut segment whose last
                                //   piece opens the chunk (b, head group, first chunk, slot
                                //   of its piece there), b = -1 if none
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t num_ranges;           // W0, workgroups
  int32_t part_units;           // most units a chunk may hold, 0 = default split
  float qk_scale_log2;          // scale * k_scale * log2(e), per-tensor scales
  float v_scale;
  const float* k_head_scales;   // [Hkv] per-head dequantisation scales, or null (per tensor):
  const float* v_head_scales;   //   kv head g then uses (qk_scale * k_head_scales[g]) * log2(e)
  float qk_scale;               // scale, for the per-head path
};

// Arguments of the merge kernels: with the default split one workgroup per chunk (the
// segment its header names), with fixed partitions one per (kv head, sequence).
struct MergeArgs {
  void* out;
  const float* rec_acc;
  const float* rec_ml;
  const int32_t* prefix;
  const int32_t* chunk_hdr;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group_waves;          // NW
  int32_t num_ranges;           // W0, decode workgroups
  int32_t part_units;
  int32_t chunk_merge;          // default split: 1 = merge_chunk_kernel, 0 = merge_kernel
  int32_t max_pieces;           // pieces a segment typically has (sizes merge_kernel)
  float v_scale;
  const float* v_head_scales;   // [Hkv] or null
};

// Multi-token queries (pa_prefill). A workgroup of kPrefillWaves waves owns one
// (sequence, kv head, tile of query tokens); each wave holds kPrefillRowGroups groups of
// 16 (token, head) rows, so a tile has 16 * kPrefillWaves * kPrefillRowGroups / G tokens.
#ifndef PA_PF_WAVES
#define PA_PF_WAVES 4
#endif
#ifndef PA_PF_ROWGROUPS
#define PA_PF_ROWGROUPS 2
#endif
constexpr int kPrefillWaves = PA_PF_WAVES;
constexpr int kPrefillRowGroups = PA_PF_ROWGROUPS;
inline int prefill_tile_tokens(int group) { return 16 * kPrefillWaves * kPrefillRowGroups / group; }

struct PrefillArgs {
  void* out;                    // [Tq, Hq, d] out dtype
  const void* q;                // [Tq, Hq, d] q dtype (16-bit)
  const void* k_pool;           // [N, 16, Hkv, d]
  const void* v_pool;
  const int32_t* block_tables;  // [B, maxb]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1]
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_query_tokens;     // Tq
  int32_t max_query_len;        // rows past it in a sequence are not computed
  int32_t num_q_tiles;          // query tiles per (sequence, kv head)
  int32_t num_workgroups;       // ceil(B * Hkv / 8) * num_q_tiles * 8
  float qk_scale_log2;          // scale * k_scale * log2(e), per-tensor scales
  float v_scale;
  const float* k_head_scales;   // [Hkv] or null: kv head g then uses
  const float* v_head_scales;   //   (qk_scale * k_head_scales[g]) * log2(e)
  float qk_scale;               // scale, for the per-head path
};

// log2(e) as a binary32 constant: host and kernels form score scales with it in the same order
constexpr float kLog2e = 1.4426950408889634f;

// Waves per workgroup for Hkv kv heads: the largest of 8, 4, 2, 1 dividing Hkv.
inline int group_waves(int num_kv_heads) {
  for (int nw = kMaxGroupWaves; nw > 1; nw >>= 1)
    if (num_kv_heads % nw == 0) return nw;
  return 1;
}

hipError_t launch_decode(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                         const DecodeArgs& args, int group_waves, hipStream_t stream);
hipError_t launch_merge(int out_dtype, int head_dim, int group, const MergeArgs& args,
                        hipStream_t stream);

// Device address of the current GPU's copy of the static decode scratch
// (PA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_prefill(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                          const PrefillArgs& args, hipStream_t stream);

hipError_t launch_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              int32_t row_bytes, int64_t num_slots, hipStream_t stream);
hipError_t launch_cache_write_fp8(void* k_pool, void* v_pool, const void* k_new,
                                  const void* v_new, const int64_t* slot_mapping,
                                  int32_t num_tokens, int32_t row_elems, int64_t num_slots,
                                  int32_t src_dtype, float k_inv, float v_inv,
                                  const float* k_head_scales, const float* v_head_scales,
                                  int32_t head_dim, hipStream_t stream);
hipError_t launch_block_copy(void* k_pool, void* v_pool, const int64_t* pairs,
                             int32_t num_pairs, int64_t block_bytes, int32_t num_blocks,
                             hipStream_t stream);
hipError_t launch_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int workgroups,
                              hipStream_t stream);
hipError_t launch_block_swap(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k,
                             const void* src_v, int32_t src_blocks, const int64_t* pairs,
                             int32_t num_pairs, int64_t block_bytes, hipStream_t stream);

}  // namespace pa
