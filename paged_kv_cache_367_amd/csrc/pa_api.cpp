// pa_api.cpp - the C ABI: argument validation, launch configuration, error codes.
//
// Every check that the host can make happens here, before anything is launched; a bad
// argument returns its pa_status_t and touches neither the GPU nor the HIP runtime.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <limits.h>

#include <atomic>

#include "../../include/paged_attention.h"
#include "pa_launch.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_dtype(int32_t d) { return d >= PA_F32 && d <= PA_FP8_E4M3; }

int dtype_bytes(int32_t d) {
  switch (d) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 1;
  }
}

bool supported_combo(int32_t q, int32_t kv, int32_t out) {
  if (q == PA_F32 && kv == PA_F32) return out == PA_F32;
  if (q == PA_F16 && kv == PA_F16) return out == PA_F16 || out == PA_F32;
  if (q == PA_BF16 && (kv == PA_BF16 || kv == PA_FP8_E4M3))
    return out == PA_BF16 || out == PA_F32;
  return false;
}

// Most workgroups a decode grid has: 8 waves per CU on at most kMaxDeviceCUs CUs, NW
// waves each. The workspace is sized for this many static chunks.
int max_workgroups(const pa_decode_desc_t* d) {
  return pa::kMaxDeviceCUs * pa::kWavesPerCU / pa::group_waves(d->num_kv_heads);
}

// Compute units of the current device (queried once per device), capped at kMaxDeviceCUs;
// kMaxDeviceCUs when the query fails.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return pa::kMaxDeviceCUs;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = pa::kMaxDeviceCUs;
    n = n < pa::kMaxDeviceCUs ? n : pa::kMaxDeviceCUs;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups of this call's decode grid: 8 waves per CU of the current device.
int num_workgroups(const pa_decode_desc_t* d) {
  return device_cus() * pa::kWavesPerCU / pa::group_waves(d->num_kv_heads);
}

// Units per chunk for an explicit partition size (0: default split).
int part_units(const pa_decode_desc_t* d) { return d->partition_size / pa::kBlockTokens; }

// Workgroups of this call's decode grid. Under the default split a call whose work is
// small (at most segments * ceil(max_context_len / 16) units) takes about two units per
// chunk rather than one chunk per workgroup of the device grid: half the pieces for the
// merge to fold, for one more unit in each workgroup's pipeline (at least 32 workgroups).
int decode_grid(const pa_decode_desc_t* d, int32_t max_context_len) {
  const int W = num_workgroups(d);
  if (part_units(d) > 0) return W;
  const int64_t seq_blocks = ((int64_t)max_context_len + pa::kBlockTokens - 1) / pa::kBlockTokens;
  const int64_t units =
      (int64_t)(d->num_kv_heads / pa::group_waves(d->num_kv_heads)) * d->batch * seq_blocks;
  const int64_t want = (units + 1) / 2;
  return want >= W ? W : (int)(want > 32 ? want : 32);
}

// Most chunks a call can have, which sizes the records in the workspace: the W static
// ones, plus with fixed partitions every partition of the largest possible unit count.
int64_t max_chunks(const pa_decode_desc_t* d, int32_t max_context_len) {
  const int W = max_workgroups(d);
  const int pu = part_units(d);
  if (pu == 0) return W;
  const int nw = pa::group_waves(d->num_kv_heads);
  const int64_t seq_blocks = ((int64_t)max_context_len + pa::kBlockTokens - 1) / pa::kBlockTokens;
  const int64_t units = (int64_t)(d->num_kv_heads / nw) * d->batch * seq_blocks;
  return (int64_t)W + (units + pu - 1) / pu;
}

pa_status_t check_desc(const pa_decode_desc_t* d, int32_t max_context_len) {
  if (!d) return PA_ERR_NULL;
  if (d->batch < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->block_size <= 0 || d->num_blocks <= 0 || d->max_blocks_per_seq <= 0 ||
      max_context_len < 0 || d->partition_size < 0)
    return PA_ERR_SHAPE;
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype) || !valid_dtype(d->out_dtype))
    return PA_ERR_DTYPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int group = d->num_q_heads / d->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (d->block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!supported_combo(d->q_dtype, d->kv_dtype, d->out_dtype)) return PA_ERR_UNSUPPORTED;
  if (d->partition_size != 0 &&
      (d->partition_size % pa::kBlockTokens != 0 || d->partition_size > pa::kMaxPartitionTokens))
    return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)d->max_blocks_per_seq * pa::kBlockTokens)
    return PA_ERR_SHAPE;
  // the batch's lengths and block prefix sums are kept in LDS
  if (d->batch > pa::kMaxBatch) return PA_ERR_UNSUPPORTED;
  // unit counts are 32-bit on the device; head groups and sequences are packed in 12 and
  // 16 bits
  const int64_t head_groups = d->num_kv_heads / pa::group_waves(d->num_kv_heads);
  if (head_groups * d->batch * d->max_blocks_per_seq > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (head_groups >= 4096) return PA_ERR_UNSUPPORTED;
  // byte offsets inside one physical block must fit 32 bits
  const int64_t block_bytes =
      (int64_t)pa::kBlockTokens * d->num_kv_heads * d->head_dim * dtype_bytes(d->kv_dtype);
  if (block_bytes > (int64_t)1 << 30) return PA_ERR_UNSUPPORTED;
  if (max_chunks(d, max_context_len) > pa::kMaxChunks) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: the records of cut segments, the per-sequence block prefix sums, then one
// 16-byte header per chunk. Every call writes what it reads, so no clearing is needed.
struct Workspace {
  size_t acc, ml, prefix, hdr, total;   // byte offsets and size
};
Workspace workspace_layout(const pa_decode_desc_t* d, int32_t max_context_len) {
  const size_t chunks = (size_t)max_chunks(d, max_context_len);
  const size_t nw = (size_t)pa::group_waves(d->num_kv_heads);
  const size_t group = (size_t)(d->num_q_heads / d->num_kv_heads);
  const size_t recs = chunks * 2 * nw * group;       // (chunk, slot, wave, q head)
  Workspace w;
  w.acc = 0;
  w.ml = w.acc + align_up(recs * d->head_dim * sizeof(float), 256);
  w.prefix = w.ml + align_up(recs * 2 * sizeof(float), 256);
  w.hdr = w.prefix + align_up(((size_t)d->batch + 1) * sizeof(int32_t), 256);
  w.total = w.hdr + align_up(chunks * 4 * sizeof(int32_t), 256);
  return w;
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return 1; }

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "invalid or inconsistent sizes";
    case PA_ERR_DTYPE: return "unknown dtype code";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PA_ERR_HIP: return "HIP runtime error at launch";
    case -8: return "not enough free or evictable KV blocks";      // pa_block_manager.h
    case -9: return "unknown sequence id, or the id is in use";   // pa_block_manager.h
    case -10: return "host memory ran out in the block manager";  // pa_block_manager.h
    case PA_ERR_SCRATCH:
      return "the call needs more workspace than pa_decode_noalloc's static scratch";
    default: return "unknown status";
  }
}

int32_t pa_decode_max_chunks(const pa_decode_desc_t* desc, int32_t max_context_len) {
  const pa_status_t st = check_desc(desc, max_context_len);
  if (st != PA_OK) return st;
  return (int32_t)max_chunks(desc, max_context_len);
}

size_t pa_decode_workspace_bytes(const pa_decode_desc_t* desc, int32_t max_context_len) {
  if (check_desc(desc, max_context_len) != PA_OK || desc->batch == 0) return 0;
  const Workspace w = workspace_layout(desc, max_context_len);
  return w.total;
}

}  // extern "C"

namespace {

// Checks of a decode call that need no workspace (PA_OK also for B = 0).
pa_status_t check_decode_call(const pa_decode_desc_t* desc, void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t max_context_len, float scale, float k_scale,
                              float v_scale) {
  pa_status_t st = check_desc(desc, max_context_len);
  if (st != PA_OK) return st;
  if (desc->batch == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale)) return PA_ERR_SHAPE;
  return PA_OK;
}

// pa_decode and pa_decode_head_scales: per-tensor scales, or (k_heads, v_heads) device
// arrays of one scale per kv head (then k_scale = v_scale = 1 here)
pa_status_t decode_impl(const pa_decode_desc_t* desc, void* out, const void* q,
                        const void* k_pool, const void* v_pool, const int32_t* block_tables,
                        const int32_t* context_lens, int32_t max_context_len, float scale,
                        float k_scale, float v_scale, const float* k_heads,
                        const float* v_heads, void* workspace, size_t workspace_bytes,
                        void* stream) {
  pa_status_t st = check_decode_call(desc, out, q, k_pool, v_pool, block_tables, context_lens,
                                     max_context_len, scale, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (desc->batch == 0) return PA_OK;
  const Workspace ws = workspace_layout(desc, max_context_len);
  if (!workspace || workspace_bytes < ws.total) return PA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  char* wsb = static_cast<char*>(workspace);
  const int nw = pa::group_waves(desc->num_kv_heads);
  const int W = decode_grid(desc, max_context_len);

  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.rec_acc = reinterpret_cast<float*>(wsb + ws.acc);
  a.rec_ml = reinterpret_cast<float*>(wsb + ws.ml);
  a.prefix = reinterpret_cast<int32_t*>(wsb + ws.prefix);
  a.chunk_hdr = reinterpret_cast<int32_t*>(wsb + ws.hdr);
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.num_blocks = desc->num_blocks;
  a.max_blocks_per_seq = desc->max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.num_ranges = W;
  a.part_units = part_units(desc);
  a.qk_scale_log2 = scale * k_scale * pa::kLog2e;
  a.v_scale = v_scale;
  a.k_head_scales = k_heads;
  a.v_head_scales = v_heads;
  a.qk_scale = scale;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int group = desc->num_q_heads / desc->num_kv_heads;
  if (pa::launch_decode(desc->q_dtype, desc->kv_dtype, desc->out_dtype, desc->head_dim, group, a,
                        nw, s) != hipSuccess)
    return PA_ERR_HIP;
  pa::MergeArgs m;
  m.out = out;
  m.rec_acc = a.rec_acc;
  m.rec_ml = a.rec_ml;
  m.prefix = a.prefix;
  m.chunk_hdr = a.chunk_hdr;
  m.batch = desc->batch;
  m.num_q_heads = desc->num_q_heads;
  m.num_kv_heads = desc->num_kv_heads;
  m.group_waves = nw;
  m.num_ranges = W;
  m.part_units = a.part_units;
  // default split: the per-chunk merge (one round trip for a segment cut once; its
  // workgroup folds longer segments alone, 8 pieces per round trip) when there are at
  // least W/4 segments and a call can have 8 units per chunk; with fewer segments or
  // units, segments tend to be cut into many pieces, and the per-(kv head, sequence)
  // merge spreads them over its workgroups, 64 per round trip
  {
    const int64_t seq_blocks =
        ((int64_t)max_context_len + pa::kBlockTokens - 1) / pa::kBlockTokens;
    const int64_t segments = (int64_t)(desc->num_kv_heads / nw) * desc->batch;
    const int64_t max_units = segments * seq_blocks;
    m.chunk_merge = (4 * segments >= W && max_units >= 8 * (int64_t)W) ? 1 : 0;
    // pieces a segment typically has (it sizes the per-segment merge's workgroups; any
    // count is handled): the chunks a call can have shared among the segments, plus one,
    // and never more than a segment's blocks
    const int64_t pu = part_units(desc);
    const int64_t chunks = pu > 0 ? W + (segments * seq_blocks + pu - 1) / pu : W;
    const int64_t pieces = (chunks + segments - 1) / (segments > 0 ? segments : 1) + 1;
    m.max_pieces = (int32_t)(pieces < seq_blocks ? pieces : seq_blocks);
  }
  m.v_scale = v_scale;
  m.v_head_scales = v_heads;
  if (pa::launch_merge(desc->out_dtype, desc->head_dim, group, m, s) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_decode(const pa_decode_desc_t* desc, void* out, const void* q,
                      const void* k_pool, const void* v_pool, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t max_context_len, float scale,
                      float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                     scale, k_scale, v_scale, nullptr, nullptr, workspace, workspace_bytes,
                     stream);
}

pa_status_t pa_decode_noalloc(const pa_decode_desc_t* desc, void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t max_context_len, float scale, float k_scale,
                              float v_scale, void* stream) {
  pa_status_t st = check_decode_call(desc, out, q, k_pool, v_pool, block_tables, context_lens,
                                     max_context_len, scale, k_scale, v_scale);
  if (st != PA_OK) return st;
  if (desc->batch == 0) return PA_OK;
  if (workspace_layout(desc, max_context_len).total > PA_NOALLOC_SCRATCH_BYTES)
    return PA_ERR_SCRATCH;
  void* ws = nullptr;
  if (pa::noalloc_scratch(&ws) != hipSuccess) return PA_ERR_HIP;
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                     scale, k_scale, v_scale, nullptr, nullptr, ws, PA_NOALLOC_SCRATCH_BYTES,
                     stream);
}

pa_status_t pa_decode_head_scales(const pa_decode_desc_t* desc, void* out, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, const float* k_scales,
                                  const float* v_scales, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (desc && desc->batch > 0 && (!k_scales || !v_scales)) return PA_ERR_NULL;
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4)) return PA_ERR_ALIGN;
  // per-head scales are built for fp8 pools (the per-head kernels are fp8 instantiations)
  if (desc && desc->kv_dtype != PA_FP8_E4M3 && valid_dtype(desc->kv_dtype))
    return PA_ERR_UNSUPPORTED;
  return decode_impl(desc, out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                     scale, 1.0f, 1.0f, k_scales, v_scales, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

pa_status_t prefill_impl(const pa_prefill_desc_t* desc, void* out, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         const int32_t* context_lens, const int32_t* query_start,
                         int32_t max_query_len, float scale, float k_scale, float v_scale,
                         const float* k_heads, const float* v_heads, void* stream) {
  const pa_prefill_desc_t* d = desc;
  if (!d) return PA_ERR_NULL;
  if (d->batch < 0 || d->num_query_tokens < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->head_dim <= 0 || d->block_size <= 0 || d->num_blocks <= 0 ||
      d->max_blocks_per_seq <= 0 || max_query_len < 0)
    return PA_ERR_SHAPE;
  if (!valid_dtype(d->q_dtype) || !valid_dtype(d->kv_dtype) || !valid_dtype(d->out_dtype))
    return PA_ERR_DTYPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_SHAPE;
  const int group = d->num_q_heads / d->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8) return PA_ERR_UNSUPPORTED;
  if (d->block_size != pa::kBlockTokens) return PA_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->kv_dtype == PA_F32 || !supported_combo(d->q_dtype, d->kv_dtype, d->out_dtype))
    return PA_ERR_UNSUPPORTED;
  if (max_query_len > d->num_query_tokens ||
      (int64_t)max_query_len > (int64_t)d->max_blocks_per_seq * pa::kBlockTokens)
    return PA_ERR_SHAPE;
  const int64_t block_bytes =
      (int64_t)pa::kBlockTokens * d->num_kv_heads * d->head_dim * dtype_bytes(d->kv_dtype);
  if (block_bytes > (int64_t)1 << 30) return PA_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->max_blocks_per_seq > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int tq = pa::prefill_tile_tokens(group);
  const int64_t tiles = ((int64_t)max_query_len + tq - 1) / tq;
  const int64_t groups = ((int64_t)d->batch * d->num_kv_heads + 7) / 8;
  if (groups * tiles * 8 > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (d->batch == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_ALIGN;
  if (!isfinite(scale) || !isfinite(k_scale) || !isfinite(v_scale)) return PA_ERR_SHAPE;

  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.batch = d->batch;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.num_blocks = d->num_blocks;
  a.max_blocks_per_seq = d->max_blocks_per_seq;
  a.num_query_tokens = d->num_query_tokens;
  a.max_query_len = max_query_len;
  a.num_q_tiles = (int32_t)tiles;
  a.num_workgroups = (int32_t)(groups * tiles * 8);
  a.qk_scale_log2 = scale * k_scale * pa::kLog2e;
  a.v_scale = v_scale;
  a.k_head_scales = k_heads;
  a.v_head_scales = v_heads;
  a.qk_scale = scale;
  if (pa::launch_prefill(d->q_dtype, d->kv_dtype, d->out_dtype, d->head_dim, group, a,
                         static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_prefill(const pa_prefill_desc_t* desc, void* out, const void* q,
                       const void* k_pool, const void* v_pool, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start,
                       int32_t max_query_len, float scale, float k_scale, float v_scale,
                       void* stream) {
  return prefill_impl(desc, out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                      max_query_len, scale, k_scale, v_scale, nullptr, nullptr, stream);
}

pa_status_t pa_prefill_head_scales(const pa_prefill_desc_t* desc, void* out, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start, int32_t max_query_len,
                                   float scale, const float* k_scales, const float* v_scales,
                                   void* stream) {
  if (desc && desc->batch > 0 && max_query_len > 0 && (!k_scales || !v_scales))
    return PA_ERR_NULL;
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4)) return PA_ERR_ALIGN;
  return prefill_impl(desc, out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                      max_query_len, scale, 1.0f, 1.0f, k_scales, v_scales, stream);
}

static pa_status_t check_cache_args(int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t kv_dtype, int64_t* row_bytes) {
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (!valid_dtype(kv_dtype)) return PA_ERR_DTYPE;
  const int64_t rb = (int64_t)num_kv_heads * head_dim * dtype_bytes(kv_dtype);
  if (rb % 16 != 0 || rb > ((int64_t)1 << 30)) return PA_ERR_UNSUPPORTED;
  *row_bytes = rb;
  return PA_OK;
}

pa_status_t pa_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t kv_dtype, void* stream) {
  int64_t row_bytes = 0;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  pa_status_t st = check_cache_args(num_kv_heads, head_dim, block_size, num_blocks, kv_dtype,
                                    &row_bytes);
  if (st != PA_OK) return st;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (pa::launch_cache_write(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                             (int32_t)row_bytes, num_slots,
                             static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // extern "C"

namespace {

pa_status_t cache_write_fp8_impl(void* k_pool, void* v_pool, const void* k_new,
                                 const void* v_new, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t src_dtype,
                                 float k_scale, float v_scale, const float* k_heads,
                                 const float* v_heads, void* stream) {
  int64_t row_bytes = 0;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  pa_status_t st = check_cache_args(num_kv_heads, head_dim, block_size, num_blocks,
                                    PA_FP8_E4M3, &row_bytes);
  if (st != PA_OK) return st;
  if (!valid_dtype(src_dtype)) return PA_ERR_DTYPE;
  if (src_dtype == PA_FP8_E4M3) return PA_ERR_UNSUPPORTED;   // use pa_cache_write
  if (!(isfinite(k_scale) && k_scale > 0.0f && isfinite(v_scale) && v_scale > 0.0f))
    return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_NULL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(slot_mapping, 8))
    return PA_ERR_ALIGN;
  // one binary32 reciprocal of each scale, rounded to nearest
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (pa::launch_cache_write_fp8(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                                 (int32_t)row_bytes, num_slots, src_dtype, k_inv, v_inv,
                                 k_heads, v_heads, head_dim,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_cache_write_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t src_dtype, float k_scale,
                               float v_scale, void* stream) {
  return cache_write_fp8_impl(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                              num_kv_heads, head_dim, block_size, num_blocks, src_dtype, k_scale,
                              v_scale, nullptr, nullptr, stream);
}

pa_status_t pa_cache_write_fp8_head_scales(void* k_pool, void* v_pool, const void* k_new,
                                           const void* v_new, const int64_t* slot_mapping,
                                           int32_t num_tokens, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t src_dtype,
                                           const float* k_scales, const float* v_scales,
                                           void* stream) {
  if (num_tokens > 0 && (!k_scales || !v_scales)) return PA_ERR_NULL;
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4)) return PA_ERR_ALIGN;
  if (head_dim % 8 != 0) return PA_ERR_UNSUPPORTED;     // an 8-value piece stays in one head
  return cache_write_fp8_impl(k_pool, v_pool, k_new, v_new, slot_mapping, num_tokens,
                              num_kv_heads, head_dim, block_size, num_blocks, src_dtype, 1.0f,
                              1.0f, k_scales, v_scales, stream);
}

pa_status_t pa_block_copy(void* k_pool, void* v_pool, const int64_t* src_dst_pairs,
                          int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                          void* stream) {
  int64_t row_bytes = 0;
  if (num_pairs < 0) return PA_ERR_SHAPE;
  pa_status_t st = check_cache_args(num_kv_heads, head_dim, block_size, num_blocks, kv_dtype,
                                    &row_bytes);
  if (st != PA_OK) return st;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_dst_pairs) return PA_ERR_NULL;
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(src_dst_pairs, 8))
    return PA_ERR_ALIGN;
  if (pa::launch_block_copy(k_pool, v_pool, src_dst_pairs, num_pairs, row_bytes * block_size,
                            num_blocks, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

pa_status_t pa_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                           void* stream) {
  if (workgroups < 0) return PA_ERR_SHAPE;
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return PA_ERR_NULL;
  if (!aligned(src, 16) || bytes % 16 != 0 || !aligned(sink, 4)) return PA_ERR_ALIGN;
  const int wg = workgroups > 0 ? workgroups : device_cus() * 8;
  if (pa::launch_stream_read(src, bytes, sink, wg, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

pa_status_t pa_block_swap(void* dst_k_pool, void* dst_v_pool, int32_t dst_num_blocks,
                          const void* src_k_pool, const void* src_v_pool, int32_t src_num_blocks,
                          const int64_t* src_dst_pairs, int32_t num_pairs, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t kv_dtype, void* stream) {
  int64_t row_bytes = 0;
  if (num_pairs < 0 || src_num_blocks <= 0) return PA_ERR_SHAPE;
  pa_status_t st = check_cache_args(num_kv_heads, head_dim, block_size, dst_num_blocks, kv_dtype,
                                    &row_bytes);
  if (st != PA_OK) return st;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k_pool || !dst_v_pool || !src_k_pool || !src_v_pool || !src_dst_pairs)
    return PA_ERR_NULL;
  if (!aligned(dst_k_pool, 16) || !aligned(dst_v_pool, 16) || !aligned(src_k_pool, 16) ||
      !aligned(src_v_pool, 16) || !aligned(src_dst_pairs, 8))
    return PA_ERR_ALIGN;
  if ((int64_t)num_pairs * 64 > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if (pa::launch_block_swap(dst_k_pool, dst_v_pool, dst_num_blocks, src_k_pool, src_v_pool,
                            src_num_blocks, src_dst_pairs, num_pairs, row_bytes * block_size,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

}  // extern "C"
