/*
 * paged_attention.h - C ABI of the paged decode-attention library (libpa.so, gfx950).
 *
 * The library implements the data-parallel hot path of PagedAttention on one MI355X:
 * decode-phase attention over a KV cache cut into fixed 16-token blocks that sit
 * anywhere in a physical pool, the slot write that stores a new token's K/V (also into
 * an fp8 cache, quantising), the block copy behind copy-on-write of shared blocks, and
 * attention of several new tokens per sequence (chunked prefill) over the same cache.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers owned by the caller (allocated with
 *     hipMalloc, or by a framework). The library allocates nothing, frees nothing and
 *     keeps no pointer after a call returns. Scalars and the descriptor are host values
 *     read during the call only.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream). Buffers must stay valid until that stream has executed the work.
 *   - Arrays are dense, row-major, no padding between rows.
 *   - Every argument the host can see is checked before anything is launched; a bad
 *     argument returns an error code and launches nothing. Errors are return codes
 *     only. Contents of device arrays (table entries, lengths, slots, pairs) are the
 *     caller's contract: kernels never read or write outside the pool for out-of-range
 *     entries (they skip them), but the result for such entries is unspecified.
 *   - No global mutable state, so calls are thread-safe; the one exception is the static
 *     per-GPU scratch of pa_decode_noalloc, whose calls must not overlap on one GPU (see
 *     there).
 */
#ifndef PAGED_ATTENTION_H
#define PAGED_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element encodings. PA_FP8_E4M3 is OCP E4M3FN (bias 7, max 448, no infinities), the
 * format behind "--kv-cache-dtype fp8" (vLLM-PagedAttention与连续批处理技术拆解,
 * section 五, flag table and the FP8 KV-cache note). */
typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3
} pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                              */
  PA_ERR_SHAPE = -2,       /* a size is negative, zero where it must not be, or sizes disagree */
  PA_ERR_DTYPE = -3,       /* unknown dtype code                                       */
  PA_ERR_UNSUPPORTED = -4, /* valid but not implemented (head_dim, group, dtype combo)   */
  PA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than pa_decode_workspace_bytes */
  PA_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned                         */
  PA_ERR_HIP = -7,         /* the HIP runtime reported an error at launch              */
  PA_ERR_SCRATCH = -11     /* pa_decode_noalloc: the call needs more than its static scratch */
} pa_status_t;

/* Shape of one decode call.
 *   batch               B, sequences (one query token each); 0 is allowed (no-op);
 *                       at most 4096, and B * max_blocks_per_seq < 2^31
 *   num_q_heads         Hq
 *   num_kv_heads        Hkv; Hq % Hkv == 0; group G = Hq / Hkv in {1, 2, 4, 8}
 *   head_dim            d in {64, 128}
 *   block_size          tokens per block; must be 16
 *   num_blocks          N, physical blocks in each pool
 *   max_blocks_per_seq  width of the block table (maxb)
 *   q_dtype, kv_dtype, out_dtype   pa_dtype_t codes; supported (q, kv, out):
 *                       (F32,F32,F32) (F16,F16,F16|F32) (BF16,BF16,BF16|F32)
 *                       (BF16,FP8_E4M3,BF16|F32)
 *   partition_size      0 (default): the KV work of the whole batch (16-token blocks of
 *                       every sequence and kv head) is cut into equal contiguous chunks,
 *                       one per workgroup of a fixed grid (8 waves per compute unit; a
 *                       smaller one, about two blocks per chunk, when the batch's
 *                       blocks at max_context_len would not fill it), whatever the length
 *                       mix; a sequence is cut only where a chunk ends. Otherwise a multiple of
 *                       16 (tokens), the split-KV partition: the work is cut into m equal
 *                       contiguous chunks per workgroup, m the smallest count for which no
 *                       chunk holds more than partition_size tokens of a sequence and kv
 *                       head, so no piece of a sequence is longer and every workgroup gets
 *                       the same work. A call whose chunks could exceed 16384 is rejected
 *                       (UNSUPPORTED). The cut points depend on the lengths only, so
 *                       results are bitwise reproducible. */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t q_dtype;
  int32_t kv_dtype;
  int32_t out_dtype;
  int32_t partition_size;
} pa_decode_desc_t;

/* Version of this ABI (1). */
int32_t pa_abi_version(void);

/* Human-readable text for a pa_status_t value; never NULL, static storage. */
const char* pa_status_string(int32_t status);

/* Most chunks (see partition_size) a call with this descriptor and max_context_len can
 * have, or a negative pa_status_t if the descriptor is invalid. */
int32_t pa_decode_max_chunks(const pa_decode_desc_t* desc, int32_t max_context_len);

/* Bytes of device workspace pa_decode needs (0 for an invalid descriptor or B = 0).
 * The workspace holds, for each chunk, the (m, l, acc) records of the at most two
 * sequence pieces it leaves unfinished (running max m in log2 units, normaliser l and
 * unnormalised output acc[d], fp32, per kv head and query head), the per-sequence prefix
 * sums of block counts, and per chunk a 16-byte header naming the sequence piece the
 * merge completes there. Every call writes what it later reads, so the workspace needs
 * no initialisation. */
size_t pa_decode_workspace_bytes(const pa_decode_desc_t* desc, int32_t max_context_len);

/* Decode attention over the paged KV cache.
 *
 * Defines: for each sequence b and query head h, with L = context_lens[b],
 * g = h / G and token t stored at k_pool[block_tables[b][t / 16]][t % 16][g][:],
 *   s_t = scale * k_scale * dot(q[b][h], K_t)          t < L
 *   out[b][h] = v_scale * sum_t softmax(s)_t * V_t
 * computed blockwise: every 16-token block contributes its local max and normaliser,
 * merged by FlashAttention-style rescaling, which equals the global softmax
 * (vLLM-PagedAttention与连续批处理技术拆解, sections 3.1-3.3; block-table lookup as in
 * the paged_attention sketch of "AI vLLM：PagedAttention不够用了之后"). A sequence
 * whose blocks span several work shares is split into pieces; each piece's (m, l, acc)
 * is merged by a second kernel with the same rescaling. Positions >= L are never
 * attended, whatever the slots hold (NaN included). L == 0 gives a zero output.
 * Two kernels are enqueued: the decode and the merge.
 *
 * Arguments (device pointers unless noted):
 *   out            [B, Hq, d] out_dtype, written
 *   q              [B, Hq, d] q_dtype
 *   k_pool, v_pool [N, 16, Hkv, d] kv_dtype (separate K and V pools)
 *   block_tables   [B, maxb] int32; entries past ceil(L/16) are ignored (-1 by convention).
 *                  An entry below ceil(L/16) outside [0, N) is a caller error; it is never
 *                  dereferenced, and its 16 tokens are left out of the softmax (the
 *                  result is the attention over the sequence's other tokens; zero if none)
 *   context_lens   [B] int32, each in [0, min(maxb*16, max_context_len)]
 *   max_context_len host int >= every context_lens[b]; sizes the launch (no device sync)
 *   scale          host float, usually 1/sqrt(d)
 *   k_scale, v_scale host floats, dequantisation scales for fp8 pools (use 1 otherwise)
 *   workspace, workspace_bytes  device scratch of at least pa_decode_workspace_bytes()
 *                  (always needed when B > 0), any contents; calls that share a
 *                  workspace must not overlap
 * All pointers must be 16-byte aligned. */
pa_status_t pa_decode(const pa_decode_desc_t* desc, void* out, const void* q,
                      const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int32_t max_context_len, float scale, float k_scale, float v_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch behind pa_decode_noalloc, one copy per GPU. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* pa_decode without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops that must
 * not call hipMalloc, harnesses that forbid it. Arguments, results and errors are those
 * of pa_decode (the same kernels run); the workspace is a static device array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library, one copy on every GPU the library runs on,
 * held until the process ends. A call whose workspace (pa_decode_workspace_bytes) would
 * exceed it returns PA_ERR_SCRATCH and launches nothing. The scratch needs no clearing
 * (every call writes what it reads), but all calls on one GPU share it: calls that overlap
 * on one GPU (on different streams, or from threads without ordering) race and give
 * undefined results; calls ordered on one stream are safe. */
pa_status_t pa_decode_noalloc(const pa_decode_desc_t* desc, void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t max_context_len, float scale, float k_scale,
                              float v_scale, void* stream);

/* Shape of one multi-token query call (pa_prefill).
 *   batch               B, sequences; 0 is allowed (no-op)
 *   num_query_tokens    Tq, query rows of all sequences together (= query_start[B])
 *   num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq
 *                       as in pa_decode_desc_t (G in {1, 2, 4, 8}, d in {64, 128},
 *                       block_size 16)
 *   q_dtype, kv_dtype, out_dtype   supported (q, kv, out): (F16,F16,F16|F32)
 *                       (BF16,BF16,BF16|F32) (BF16,FP8_E4M3,BF16|F32); fp32 K/V is not
 *                       supported here (UNSUPPORTED) */
typedef struct {
  int32_t batch;
  int32_t num_query_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t q_dtype;
  int32_t kv_dtype;
  int32_t out_dtype;
} pa_prefill_desc_t;

/* Attention of several new query tokens per sequence over the paged KV cache: the
 * kernel side of chunked prefill (a long prompt prefilled a chunk per step) and of a
 * prefix-cache hit that prefills only the uncached tail (LLM KV cache serving-engine
 * article, sections 3 and 4). The new tokens' K/V must already be in the cache (slot
 * write first).
 *
 * Defines: sequence b has L = context_lens[b] cached tokens, the last
 * n = query_start[b+1] - query_start[b] of which are its query tokens; query token i
 * (row query_start[b] + i of q and out) sits at position p = L - n + i and, for each query
 * head h (kv head g = h / G),
 *   s_t = scale * k_scale * dot(q[row][h], K_t)           0 <= t <= p
 *   out[row][h] = v_scale * sum_t softmax(s)_t * V_t
 * with the blockwise softmax merge of pa_decode (n = 1 is a decode step). Rows with p < 0
 * (n > L) attend over nothing and are zero. Positions >= L are never read into the
 * result, whatever the slots hold.
 *
 * Arguments (device pointers unless noted):
 *   out            [Tq, Hq, d] out_dtype, written for the first min(n, max_query_len)
 *                  rows of each sequence
 *   q              [Tq, Hq, d] q_dtype
 *   k_pool, v_pool [N, 16, Hkv, d] kv_dtype
 *   block_tables   [B, maxb] int32; entries past ceil(L/16) are ignored; an entry below it
 *                  outside [0, N) is never read and its 16 positions are left out of
 *                  every row's softmax (a caller error, as for pa_decode)
 *   context_lens   [B] int32, each in [0, maxb*16] (larger values are clamped)
 *   query_start    [B + 1] int32, non-decreasing from 0 to Tq
 *   max_query_len  host int >= every n; sizes the launch (no device sync); at most
 *                  min(Tq, maxb*16)
 *   scale, k_scale, v_scale   host floats, as for pa_decode
 * No workspace. One kernel is enqueued. All pointers must be 16-byte aligned (the int32
 * arrays 4-byte). */
pa_status_t pa_prefill(const pa_prefill_desc_t* desc, void* out, const void* q,
                       const void* k_pool, const void* v_pool, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start,
                       int32_t max_query_len, float scale, float k_scale, float v_scale,
                       void* stream);

/* Per-head dequantisation scales (the fp8 KV cache row's "per-head scales"): the same as
 * pa_decode and pa_prefill, except that kv head g's K codes are multiplied by k_scales[g]
 * and its V codes by v_scales[g] instead of one k_scale / v_scale for the whole pool.
 * k_scales, v_scales: DEVICE arrays of Hkv floats (finite and > 0: the caller's contract;
 * the library cannot check device values), 4-byte aligned; required (non-NULL) whenever the
 * call has work. pa_decode_head_scales takes fp8 E4M3 pools only (other kv dtypes:
 * UNSUPPORTED); pa_prefill_head_scales any supported kv dtype. With all scales equal the
 * results are bitwise those of the per-tensor calls. */
pa_status_t pa_decode_head_scales(const pa_decode_desc_t* desc, void* out, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t max_context_len, float scale, const float* k_scales,
                                  const float* v_scales, void* workspace,
                                  size_t workspace_bytes, void* stream);
pa_status_t pa_prefill_head_scales(const pa_prefill_desc_t* desc, void* out, const void* q,
                                   const void* k_pool, const void* v_pool,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* query_start, int32_t max_query_len,
                                   float scale, const float* k_scales, const float* v_scales,
                                   void* stream);

/* Slot write of new tokens (reshape_and_cache): a generated token occupies one slot
 * (vLLM-PagedAttention与连续批处理技术拆解, section 3.1). For each t < num_tokens with
 * slot_mapping[t] = s >= 0:
 *   k_pool[s / block_size][s % block_size][:][:] = k_new[t][:][:]   (and V likewise)
 * a bit-exact copy in the pool's encoding. s < 0 skips the token; slots must be
 * distinct and < num_blocks * block_size (out-of-range slots are skipped).
 *   k_pool, v_pool [N, block_size, Hkv, d]; k_new, v_new [T, Hkv, d]; slot_mapping [T]
 *   int64. Hkv * d * bytes(kv_dtype) must be a multiple of 16. */
pa_status_t pa_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                           const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t kv_dtype, void* stream);

/* Slot write into an fp8 E4M3 cache, quantising the new values (setting the KV cache to
 * fp8 E4M3 halves its memory: vLLM-PagedAttention与连续批处理技术拆解, section 五, the
 * flag table and the KV cache quantisation note). For each t < num_tokens with
 * slot_mapping[t] = s >= 0 and every element x of k_new[t] (of v_new[t] with v_scale):
 *   y = fp32(x) * fp32(1 / k_scale)          one binary32 multiply, round to nearest even
 *   k_pool byte = E4M3FN(y)                  nearest value, ties to the even mantissa;
 *                                            |y| >= 448 (and +-inf) saturate to +-448;
 *                                            NaN -> 0x7F; the sign of zero is kept
 * so that decoding code * k_scale (pa_decode's k_scale) approximates x. Pools are OCP
 * E4M3FN bytes [N, block_size, Hkv, d]; k_new, v_new [T, Hkv, d] in src_dtype (PA_F32,
 * PA_F16 or PA_BF16; PA_FP8_E4M3 sources use pa_cache_write); slot_mapping [T] int64,
 * as for pa_cache_write (s < 0 skips, out-of-range slots are skipped). k_scale and
 * v_scale must be finite and > 0 (else PA_ERR_SHAPE); Hkv * d must be a multiple of 16.
 * fp32 subnormal inputs may be flushed to zero of either sign by the hardware conversion
 * (they lie far below E4M3's smallest value, 2^-9, and encode as zero). */
pa_status_t pa_cache_write_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t src_dtype, float k_scale,
                               float v_scale, void* stream);

/* The same with one scale per kv head: element x of kv head g quantises with
 * y = fp32(x) * fp32(1 / k_scales[g]) (the reciprocal rounded to nearest, as the host
 * rounds it for pa_cache_write_fp8), V likewise with v_scales[g]. k_scales, v_scales:
 * DEVICE arrays of Hkv floats, finite and > 0 (caller's contract), 4-byte aligned, required
 * when num_tokens > 0; head_dim must be a multiple of 8 (else UNSUPPORTED). */
pa_status_t pa_cache_write_fp8_head_scales(void* k_pool, void* v_pool, const void* k_new,
                                           const void* v_new, const int64_t* slot_mapping,
                                           int32_t num_tokens, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size,
                                           int32_t num_blocks, int32_t src_dtype,
                                           const float* k_scales, const float* v_scales,
                                           void* stream);

/* Copy-on-write block copy: a shared block is read-only and a sequence that must write
 * into it copies it first (vLLM-PagedAttention与连续批处理技术拆解, section 3.4). For
 * each pair p: k_pool[dst_p] = k_pool[src_p] and v_pool[dst_p] = v_pool[src_p], whole
 * blocks (block_size x Hkv x d), bit-exact.
 *   src_dst_pairs [P, 2] int64 (src, dst). Destinations must be distinct and no
 *   destination may be a source in the same call; pairs with an id outside [0, N) are
 *   skipped. */
pa_status_t pa_block_copy(void* k_pool, void* v_pool, const int64_t* src_dst_pairs,
                          int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, int32_t kv_dtype,
                          void* stream);

/* Block swap between two pools (preemption by swapping: a victim sequence's blocks move to
 * host memory and come back later; vLLM-PagedAttention与连续批处理技术拆解, section 4.3). For
 * each pair p: dst_k_pool[dst_p] = src_k_pool[src_p] and dst_v_pool[dst_p] =
 * src_v_pool[src_p], whole blocks (block_size x Hkv x d), bit-exact, one launch for all
 * pairs. Either pool may be device memory or pinned host memory (hipHostMalloc); the pairs
 * [P, 2] int64 (src block in the source pool, dst block in the destination pool) must be
 * device-accessible (device memory or pinned host memory). The pools must not overlap and
 * destinations must be distinct; pairs with an id outside [0, src_num_blocks) or
 * [0, dst_num_blocks) are skipped. Sizes as for pa_block_copy (num_blocks there is
 * dst_num_blocks here); P * 64 < 2^31. */
pa_status_t pa_block_swap(void* dst_k_pool, void* dst_v_pool, int32_t dst_num_blocks,
                          const void* src_k_pool, const void* src_v_pool, int32_t src_num_blocks,
                          const int64_t* src_dst_pairs, int32_t num_pairs, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t kv_dtype, void* stream);

/* Measurement aid, not part of the attention path: reads `bytes` of device memory at `src`
 * once (each of `workgroups` workgroups of 256 threads streams a contiguous slab with
 * eight 16-byte non-temporal loads in flight per thread; 0 = 8 workgroups per compute
 * unit) and writes at most one 32-bit word to `sink`, so that its time
 * gives the read-only HBM bandwidth that a kernel which only reads (the decode) can reach
 * on this GPU. src and sink are device pointers, src 16-byte aligned, bytes a multiple of
 * 16. */
pa_status_t pa_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTENTION_H */
