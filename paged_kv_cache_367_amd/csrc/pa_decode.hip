// pa_decode.hip - decode attention over a block-paged KV cache, gfx950 (CDNA4).
//
// What is computed (vLLM-PagedAttention与连续批处理技术拆解, sections 3.1-3.3): every
// sequence's single query attends over its first L tokens, whose K/V rows live in
// 16-token blocks found through the sequence's block table. Softmax is computed block
// by block: each block contributes its local max and normaliser, and running results
// are rescaled whenever the max moves (FlashAttention-style), which equals the global
// softmax exactly in real arithmetic. A long sequence is split into pieces whose
// (max, normaliser, output) triples are merged the same way.
//
// How it maps onto CDNA4
//   * Persistent, balanced work split. A unit is one 16-token block of one sequence for
//     one head group of NW kv heads (NW = 8 when Hkv allows). Units are numbered
//     sequence by sequence; a fixed grid of W workgroups (8 waves per CU of the device)
//     takes equal contiguous shares, whatever the length mix. Wave w of a workgroup
//     handles kv head hg*NW + w, so the NW waves read the NW head slices of the same
//     blocks at the same time: each token row is read as one contiguous stretch.
//   * Each wave streams its share as one pipeline over sequence boundaries: step s
//     computes unit s while the K/V loads of the next NBUF units and the block-id loads
//     of the NBUF after those are in flight. K/V loads are raw buffer loads from a
//     per-block scalar descriptor; a unit past the share gets an empty descriptor, so
//     the instruction stream (and every wait count) is the same at every step.
//   * 16-bit and fp8 K/V: scores are computed as K.Q^T on the matrix cores
//     (v_mfma_f32_16x16x32_{bf16,f16}; fp8 is widened exactly to bf16 first). Operand A
//     is the K block exactly as it sits in HBM: lane (t, q) = (lane % 16, lane / 16) loads
//     16-byte chunk 4s+q of token t's row. fp8 K, whose row of one kv head is a single
//     128-byte line, goes through LDS instead: loads that each take whole rows (8 lanes per
//     row) write a per-slot LDS ring directly (buffer loads with the lds bit, chunks
//     XOR-swizzled by row), and each unit's operand is read back from there one unit
//     ahead; half-line loads cost the fp8 path 3%. Operand B repeats the G query rows over the 16
//     MFMA columns (column n holds head n % G), laid out once per piece through LDS. The
//     MFMA's output leaves lane (n, kq) with the scores of tokens 4kq .. 4kq+3 for head
//     n % G, which is the A-operand layout of P in P.V, so P never leaves registers.
//   * Block max: in-lane over the 4 tokens, then v_permlane16/32_swap across the 4 row
//     groups; the running (m, l) and the rescale of the accumulators stay in registers.
//   * P.V on the matrix cores (v_mfma_f32_16x16x32 in the K/V element type): the 32-deep
//     contraction takes the 16-bit hi part and the 16-bit lo part of every weight p against
//     the same V row, so the weights enter within 2^-16 of their fp32 value; l sums the
//     fp32 weights. Lane (n, kq) loads dims D/16*n .. of tokens 4kq .. 4kq+3; the B operand
//     is two byte permutes away (fp8: one byte permute per two dims interleaves two tokens
//     before the conversions, which then give B operand halves directly).
//   * fp32 K/V: QK^T on v_mfma_f32_16x16x4f32, p through LDS, and P.V on the vector ALU in
//     fp32: lane (r, c) owns V chunk c of rows r, r + RPI, ... for all G heads; lanes
//     owning the same chunk are summed at the end of a piece.
//   * A sequence whose segment lies in one share is written out directly. A segment cut
//     by share boundaries leaves one (m, l, acc) record per piece (at most two per wave:
//     the share's first and last segment), and a merge kernel combines them
//     (merge_chunk_kernel: one workgroup per chunk, named by a header the decode
//     writes; with fixed partitions merge_kernel, one per (kv head, sequence)). With
//     fixed partitions a workgroup takes a contiguous run of partitions, assigned
//     statically from the lengths.
//   * The partial last block is masked by selection (scores -> -inf, V rows read as 0), so
//     stale or NaN slots past L never reach the result. A block id outside the pool is
//     never dereferenced; its 16 tokens are masked the same way.
//   * Reduction order depends on logical positions and lengths only, never on physical
//     block ids, so moving blocks in the pool leaves the output bitwise unchanged.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/paged_attention.h"
#include "pa_device.h"
#include "pa_launch.h"

// Workspace of pa_decode_noalloc: one copy per GPU for the life of the process. In host
// code this name stands for the device symbol only; kernels get the device address that
// noalloc_scratch looks up.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa {
namespace {

#ifndef PA_RING_BYTES
#define PA_RING_BYTES 16384
#endif
constexpr int kRingBytes = PA_RING_BYTES;  // K and V bytes in flight per wave (ring depth)

// Row reductions use four DPP steps, quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror and row_mirror: after them every lane of a 16-lane row holds the
// row's result.
//
// Row maxima of N independent values per lane (N = 1, 2, 4), in place: v_max_f32 with a
// DPP source over the same four steps. The N chains are interleaved so that each DPP
// source was written at least two wait states earlier (s_nop fills the rest), and the
// fused form skips the separate move and the NaN-quieting max the compiler adds.
#define PA_DPPMAX(i, ctl) "v_max_f32_dpp %" #i ", %" #i ", %" #i " " ctl " row_mask:0xf bank_mask:0xf\n"
#define PA_Q1 "quad_perm:[1,0,3,2]"
#define PA_Q2 "quad_perm:[2,3,0,1]"
#define PA_HM "row_half_mirror"
#define PA_MI "row_mirror"
template <int N>
__device__ __forceinline__ void row16_max_n(float (&x)[N]) {
  static_assert(N == 1 || N == 2 || N == 4, "1, 2 or 4 rows");
  if constexpr (N == 4) {
    asm volatile("s_nop 1\n"
                 PA_DPPMAX(0, PA_Q1) PA_DPPMAX(1, PA_Q1) PA_DPPMAX(2, PA_Q1) PA_DPPMAX(3, PA_Q1)
                 PA_DPPMAX(0, PA_Q2) PA_DPPMAX(1, PA_Q2) PA_DPPMAX(2, PA_Q2) PA_DPPMAX(3, PA_Q2)
                 PA_DPPMAX(0, PA_HM) PA_DPPMAX(1, PA_HM) PA_DPPMAX(2, PA_HM) PA_DPPMAX(3, PA_HM)
                 PA_DPPMAX(0, PA_MI) PA_DPPMAX(1, PA_MI) PA_DPPMAX(2, PA_MI) PA_DPPMAX(3, PA_MI)
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
  } else if constexpr (N == 2) {
    asm volatile("s_nop 1\n"
                 PA_DPPMAX(0, PA_Q1) PA_DPPMAX(1, PA_Q1) "s_nop 0\n"
                 PA_DPPMAX(0, PA_Q2) PA_DPPMAX(1, PA_Q2) "s_nop 0\n"
                 PA_DPPMAX(0, PA_HM) PA_DPPMAX(1, PA_HM) "s_nop 0\n"
                 PA_DPPMAX(0, PA_MI) PA_DPPMAX(1, PA_MI)
                 : "+v"(x[0]), "+v"(x[1]));
  } else {
    asm volatile("s_nop 1\n" PA_DPPMAX(0, PA_Q1) "s_nop 1\n" PA_DPPMAX(0, PA_Q2)
                 "s_nop 1\n" PA_DPPMAX(0, PA_HM) "s_nop 1\n" PA_DPPMAX(0, PA_MI)
                 : "+v"(x[0]));
  }
}
#undef PA_DPPMAX
#undef PA_Q1
#undef PA_Q2
#undef PA_HM
#undef PA_MI
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Matrix-core P.V (16-bit K/V). V words of one token row, as pairs of 16-bit values in the
// MFMA's element type.
template <int KV, int WORDS, typename VTy>
__device__ __forceinline__ void v_words16(const VTy& w, uint32_t (&o)[WORDS]) {
  static_assert(KV == PA_F16 || KV == PA_BF16, "16-bit V");
#pragma unroll
  for (int i = 0; i < WORDS; ++i) o[i] = w[i];
}
// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l
// writes lds + 16 l; a lane whose offset is out of range writes zeros.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}
// Matrix-core path: scores as K.Q^T, so that the MFMA's output layout (lane (n, kq): rows
// 4kq + v, column n) gives each lane tokens 4kq .. 4kq+3 of head n % G, which is the A
// operand layout P takes in P.V. One 16-byte K chunk (A) against the matching q piece(s)
// (B): acc += A(k) * B(q).
template <int KV>
__device__ __forceinline__ f32x4 kq_chunk(f32x4 acc, u32x4 k, const u32x4* qc) {
  if constexpr (KV == PA_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                  __builtin_bit_cast(bf16x8, qc[0]), acc, 0, 0, 0);
  } else if constexpr (KV == PA_F16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                 __builtin_bit_cast(f16x8, qc[0]), acc, 0, 0, 0);
  } else {
    static_assert(KV == PA_FP8_E4M3, "16-bit and fp8 K only");
    // 16 E4M3 values -> two groups of 8 bf16 (exact: every E4M3 value is a bf16 value)
    bf16x2 e[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      e[2 * w] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.0f, false);
      e[2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.0f, true);
    }
    bf16x8 k0 = {e[0][0], e[0][1], e[1][0], e[1][1], e[2][0], e[2][1], e[3][0], e[3][1]};
    bf16x8 k1 = {e[4][0], e[4][1], e[5][0], e[5][1], e[6][0], e[6][1], e[7][0], e[7][1]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, __builtin_bit_cast(bf16x8, qc[0]), acc,
                                                  0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, __builtin_bit_cast(bf16x8, qc[1]), acc,
                                                  0, 0, 0);
  }
  return acc;
}
// p of four tokens as the A operand of a 16x16x32 P.V MFMA: elements 0..3 hold hi(p) of
// tokens 4kq .. 4kq+3 and elements 4..7 lo(p), the remainder p - hi(p) in the same 16-bit
// type; the B operand repeats the four V rows, so the product takes sum (hi + lo) v. bf16:
// hi is p with its low 16 bits cleared (exact, relative error below 2^-7), lo that
// remainder rounded to nearest even, so hi + lo is p to within 2^-16 relative. fp16: hi
// and lo rounded to nearest even (within 2^-22).
template <int KV>
__device__ __forceinline__ u32x4 split_pack4(const float (&p)[4]) {
  u32x4 a;
  if constexpr (KV == PA_F16) {
    _Float16 h[4], l[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      h[v] = (_Float16)p[v];
      l[v] = (_Float16)(p[v] - (float)h[v]);
    }
    auto pk = [](_Float16 x, _Float16 y) {
      return (uint32_t)__builtin_bit_cast(uint16_t, x) |
             (uint32_t)__builtin_bit_cast(uint16_t, y) << 16;
    };
    a[0] = pk(h[0], h[1]);
    a[1] = pk(h[2], h[3]);
    a[2] = pk(l[0], l[1]);
    a[3] = pk(l[2], l[3]);
  } else {
    uint32_t b[4];
    float r[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      b[v] = __float_as_uint(p[v]);
      r[v] = p[v] - __uint_as_float(b[v] & 0xffff0000u);   // exact
    }
    a[0] = __builtin_amdgcn_perm(b[1], b[0], 0x07060302u);   // upper halves of p0, p1
    a[1] = __builtin_amdgcn_perm(b[3], b[2], 0x07060302u);
    const bf16x2 l01 = {(__bf16)r[0], (__bf16)r[1]}, l23 = {(__bf16)r[2], (__bf16)r[3]};
    a[2] = __builtin_bit_cast(uint32_t, l01);
    a[3] = __builtin_bit_cast(uint32_t, l23);
  }
  return a;
}
// P.V on a 16x16x32 MFMA in the element type of KV (fp16 for fp16, bf16 otherwise): the
// A operand from split_pack4, the B operand the lane's four V values (two words) twice.
template <int KV>
__device__ __forceinline__ f32x4 mfma_pv(u32x4 a, u32x2 b, f32x4 c) {
  const u32x4 bb = {b[0], b[1], b[0], b[1]};
  if constexpr (KV == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, bb), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, bb), c, 0, 0, 0);
}
// DPP quad broadcast: every lane gets the value of lane I of its quad
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return dpp<I * 0x55>(x);
}

// Vector-ALU path (fp32 K/V): one 16-byte K chunk against the matching q piece:
// acc += A(q) * B(k), four 16x16x4 fp32 MFMAs.
__device__ __forceinline__ f32x4 qk_chunk_f32(f32x4 acc, u32x4 k, const u32x4* qc) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qc[0][e]), __uint_as_float(k[e]),
                                               acc, 0, 0, 0);
  return acc;
}

// Context length clamped to [0, cap]; cap = min(table width * 16, max_context_len).
__device__ __forceinline__ int clamp_len(int L, int cap) {
  L = L < 0 ? 0 : L;
  return L < cap ? L : cap;
}
__device__ __forceinline__ int nblocks(int L) { return (L + kBlockTokens - 1) / kBlockTokens; }

// Full-wave reductions (xor butterfly over all 64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int st = 1; st < kWave; st <<= 1) x = fmaxf(x, __shfl_xor(x, st));
  return x;
}

// Register allocation target: 8 waves per CU (2 per SIMD), i.e. at most 256 VGPRs.
constexpr int kMaxThreads = kMaxGroupWaves * kWave;

// Per-unit bookkeeping carried (in scalar registers) from the id fetch to the K/V issue
// to the compute stage.
// Unit flags: valid; first / last unit of a piece (the part of a segment inside one
// chunk); the piece starts its chunk; the unit is the first / last block of its segment.
enum : int { kValid = 1, kFirst = 2, kLast = 4, kAtStart = 8, kSegStart = 16, kSegEnd = 32 };
// Packed so that the ring's bookkeeping stays in a few scalar registers:
//   bf = b | flags << 16 | rem << 24   (rem: tokens of the block below L, 1..16)
//   hc = head group | chunk << 12
struct UnitMeta {
  int bf, j, hc;
  __device__ int b() const { return bf & 0xffff; }
  __device__ int flags() const { return (bf >> 16) & 0xff; }
  __device__ int rem() const { return bf >> 24; }
  __device__ int hg() const { return hc & 0xfff; }
  __device__ int chunk() const { return hc >> 12; }
};

// PH: per-head dequantisation scales (k_head_scales / v_head_scales); a separate
// instantiation, so the per-tensor kernels carry no extra registers.
template <int KV, int QT, int OT, int D, int G, bool PH>
__global__ __launch_bounds__(kMaxThreads, 1) void decode_kernel(DecodeArgs a) {
  constexpr int KB = Enc<KV>::bytes;
  constexpr int QB = Enc<QT>::bytes;
  constexpr int ROWB = D * KB;            // bytes of one token's K (or V) row, one kv head
  constexpr int NL = ROWB / 64;           // K: 16-byte loads per lane per block
  constexpr int EPC = 16 / KB;            // K: elements per 16-byte chunk
  // P.V runs on the matrix cores for 16-bit and fp8 K/V (MPV): lane (n, kq) = (lane % 16,
  // lane / 16) loads DPL dims (DPL*n ..) of tokens 4kq .. 4kq+3, one token per load, so
  // the 16x16x16 MFMA's B operand for dim DPL*n + e is two byte permutes away. fp32 K/V
  // keeps P.V on the vector ALU: lane (r, c) loads 16-byte chunk c of rows r, r + RPI, ...
  constexpr bool MPV = KV != PA_F32;
  constexpr int DPL = D / 16;
  constexpr int VB = MPV ? DPL * KB : 16;  // V bytes per lane per load
  constexpr int VEPC = VB / KB;            // V elements per lane per load
  constexpr int LPR = MPV ? 16 : ROWB / VB;
  constexpr int RPI = kWave / LPR;
  constexpr int NLV = kBlockTokens / RPI; // V: loads per lane per block
  using VT = typename VChunk<VB>::type;
  constexpr int QROWS = G > 4 ? G / 4 : 1;  // MFMA row groups holding distinct heads
  constexpr int HPL = G < 4 ? G : 4;        // distinct heads per lane after the MFMA
  constexpr int QCH = EPC * QB / 16;        // 16-byte q pieces matching one K chunk
  constexpr int QBYTES = G * D * QB;        // the G query rows of one (sequence, kv head)
  constexpr int QPL = (QBYTES + kWave * 16 - 1) / (kWave * 16);  // q pieces per lane
  static_assert(NL >= 1 && LPR <= kWave && NLV * RPI == kBlockTokens, "block layout");
  static_assert(QCH >= 1, "q layout");
  // ring depth NBUF (units in flight while one more is computed): about kRingBytes of
  // K and V per wave, at most 3, and few enough that the R = NBUF + 1 register slots fit
  // the 256 registers of 2 waves per SIMD next to the accumulators and q operand
  constexpr int BLK_WAVE_BYTES = (NL * 16 + NLV * VB) * kWave;  // K + V of one block, one wave
  constexpr int SLOT_VGPRS = NL * 4 + NLV * (VB / 4) + QPL * 4 + 1;
  constexpr int FIXED_VGPRS = (MPV ? DPL * 4 : G * VEPC) + NL * QCH * 4 + 2 * G + 80;
  constexpr int NBUF_FIT = (256 - FIXED_VGPRS) / SLOT_VGPRS - 1;
  constexpr int NBUF_BYTES = kRingBytes / BLK_WAVE_BYTES;
  constexpr int NBUF_MIN = NBUF_BYTES < NBUF_FIT ? NBUF_BYTES : NBUF_FIT;
#ifdef PA_NBUF
  constexpr int NBUF = PA_NBUF;
#else
  constexpr int NBUF = NBUF_MIN < 1 ? 1 : (NBUF_MIN > 3 ? 3 : NBUF_MIN);
#endif
  constexpr int PBUF = kBlockTokens * G + 8;    // p of one block (+ alpha[8]), one wave

  __shared__ int s_lens[kMaxBatch];        // clamped context length per sequence
  __shared__ int s_first[kMaxBatch];       // first block id of each sequence
  __shared__ uint8_t s_shr[kMaxBatch];     // the sequence probably shares blocks
  __shared__ int s_pre[kMaxBatch + 1];     // blocks before each sequence
  __shared__ int s_wsum[kMaxGroupWaves];
  __shared__ float s_p[kMaxGroupWaves][2 * PBUF];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[kMaxGroupWaves][QBYTES];
  // fp8 K (KLDS): each ring slot's K blocks, one per wave, loaded whole token rows at a
  // time straight into LDS and read back in the matrix-core operand layout; one array per
  // slot, so that reading a slot waits only for that slot's loads
  constexpr bool KLDS = KV == PA_FP8_E4M3;
  constexpr int KBLK = kBlockTokens * ROWB;            // K bytes of one block, one kv head
  constexpr int KR_BYTES = KLDS ? kMaxGroupWaves * KBLK : 16;
  __shared__ __attribute__((aligned(16))) uint8_t s_kr0[KR_BYTES], s_kr1[KR_BYTES],
      s_kr2[KR_BYTES], s_kr3[KR_BYTES];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int nthr = blockDim.x;
  const int NW = nthr / kWave;
  // uniform within a wave; say so, so that everything derived stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int B = a.batch, Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int HGC = uni(Hkv / NW);                     // head groups
  const int cap = min(a.max_blocks_per_seq * kBlockTokens, a.max_context_len);

  // ---- 1. lengths and block prefix sums of the whole batch, in LDS. Thread t owns the
  // sequences [t*K, t*K + K). Every workgroup computes them; workgroup 0 also stores the
  // prefix sums for the merge. The first block id of every sequence rides along (same
  // memory round trip): a sequence whose first block is its neighbour's (parallel samples
  // or beam forks of one prompt) shares blocks, and so does every sequence of a batch
  // that references more blocks than the pool holds. A workgroup that visits such a
  // sequence keeps the cached policy for its K/V loads, so that the other readers of a
  // shared block find it in the caches; the others stream K/V, read once, past them.
  const int K = (B + nthr - 1) / nthr;
  const int b_lo = min(B, tid * K), b_hi = min(B, b_lo + K);
  int mine = 0;
  for (int b = b_lo; b < b_hi; ++b) {
    const int L = clamp_len(a.context_lens[b], cap);
    const int f = a.block_tables[(size_t)b * a.max_blocks_per_seq];
    s_lens[b] = L;
    s_first[b] = L > 0 ? f : -1 - b;        // distinct from every id when empty
    mine += nblocks(L);
  }
  int incl = mine;
#pragma unroll
  for (int st = 1; st < kWave; st <<= 1) {
    const int y = __shfl_up(incl, st);
    if (lane >= st) incl += y;
  }
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < NW; ++w) {
    const int x = uni(s_wsum[w]);
    before += w < wave ? x : 0;
    total += x;
  }
  {
    const bool oversubscribed = total > a.num_blocks;
    int c = before + incl - mine;                    // blocks of sequences before b_lo
    for (int b = b_lo; b < b_hi; ++b) {
      s_pre[b] = c;
      if (blockIdx.x == 0) a.prefix[b] = c;
      c += nblocks(s_lens[b]);
      const int f = s_first[b];
      s_shr[b] = oversubscribed || (b > 0 && s_first[b - 1] == f) ||
                 (b + 1 < B && s_first[b + 1] == f);
    }
    if (tid == 0) {
      s_pre[B] = total;
      if (blockIdx.x == 0) a.prefix[B] = total;
    }
  }

  // ---- 2. chunks. T units in W equal static chunks, m per workgroup (m = 1 by default;
  // with fixed partitions just enough that no chunk exceeds the partition). Workgroup r
  // takes chunks r*m .. r*m + m - 1, the r dealt to the 8 XCDs in contiguous eighths
  // (workgroups go to XCDs round-robin) so that neighbouring sequences share an L2.
  const int W0 = a.num_ranges, bid = blockIdx.x;
  const ChunkGeom cg = chunk_geometry((int64_t)HGC * total, W0, a.part_units);
  const int W = cg.W;
  const int rng = (W0 % 8 == 0) ? (bid % 8) * (W0 / 8) + bid / 8 : bid;
  const int c_last = rng * cg.per_wg + cg.per_wg - 1;
  __syncthreads();

  // ---- 3. the unit walker (scalar): position in the current chunk, sequence, head
  // group, block
  int cur = -1;                              // current chunk, -1 once there is none
  int wu = 0, cbeg = 0, cend = 0;
  int wb = 0, whg = 0, wj = 0, wnb = 1, wL = 0;
  // largest b with HGC * pre[b] <= u (the sequence holding unit u: empty sequences
  // before it share its prefix sum). The prefix sums never decrease, so the b passing the
  // test form a prefix of [0, B): count them with two wave ballots, first over 64 evenly
  // spaced samples, then inside the stretch the count ends in.
  const int SPAN = (B + kWave - 1) / kWave;
  auto seq_of = [&](int u) -> int {
    const int b1 = lane * SPAN;
    const bool p1 = b1 < B && HGC * s_pre[b1] <= u;
    const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(p1)) - 1;
    const int b2 = k * SPAN + lane;
    const bool p2 = lane < SPAN && b2 < B && HGC * s_pre[b2] <= u;
    return uni(k * SPAN + __builtin_popcountll(__builtin_amdgcn_ballot_w64(p2)) - 1);
  };
  auto locate = [&](int u) {
    const int lo = seq_of(u);
    wb = lo;
    wL = uni(s_lens[lo]);
    wnb = nblocks(wL);
    const int rel = u - HGC * uni(s_pre[lo]);
    whg = uni(rel / wnb);   // integer division runs on the vector ALU
    wj = rel - whg * wnb;
  };
  // Header of the static chunk for merge_chunk_kernel (default split only): the segment
  // whose last piece opens the chunk, if it began in an earlier chunk. Noted at entry,
  // written once the first loads are in flight (its divisions are then off the path to
  // the first data).
  int hdr_c = -1, hdr_b = -1, hdr_hg = 0, hdr_sseg = 0;
  auto note_header = [&](int c, bool cut, int sseg) {
    hdr_c = c;
    hdr_b = cut ? wb : -1;
    hdr_hg = whg;
    hdr_sseg = sseg;
  };
  auto enter = [&](int c) {
    cur = c;
    if (c < 0) return;
    cbeg = uni((int)chunk_begin(cg, c));
    cend = uni((int)chunk_end(cg, c));
    wu = cbeg;
    locate(wu);
    if (!cg.fixed) {
      const int sseg = HGC * uni(s_pre[wb]) + whg * wnb;
      note_header(c, wj > 0 && sseg + wnb <= cend, sseg);
    }
  };
  // the workgroup's first non-empty chunk after c, or -1
  auto next_nonempty = [&](int c) {
    for (++c; c <= c_last; ++c)
      if (chunk_begin(cg, c) < chunk_end(cg, c)) return c;
    return -1;
  };
  // at a chunk end: the workgroup's next chunk, or none
  auto next_chunk = [&]() { enter(next_nonempty(cur)); };
  if (!cg.fixed && chunk_begin(cg, rng) == chunk_end(cg, rng))
    note_header(rng, false, 0);   // an empty chunk ends no segment
  enter(next_nonempty(rng * cg.per_wg - 1));
  // the workgroup's K/V loads keep the cached policy when any sequence it visits probably
  // shares blocks, and stream otherwise (decided once, so the loop carries no branch)
  bool wg_shared = false;
  if (cur >= 0) {
    const int b_last = seq_of((int)chunk_end(cg, c_last) - 1);
    bool any = false;
    for (int b = wb + lane; b <= b_last; b += kWave) any |= s_shr[b] != 0;
    wg_shared = __builtin_amdgcn_ballot_w64(any) != 0;
  }
  // default split: sequences of length 0 own no units; workgroup r writes the zero
  // outputs of sequences r, r + W, ... (with fixed partitions the merge does)
  if (!cg.fixed) {
    const size_t row = (size_t)Hq * D;
    for (int b = bid; b < B; b += W)
      if (s_lens[b] == 0)
        for (size_t i = tid; i < row; i += nthr) store_out<OT>(a.out, (size_t)b * row + i, 0.0f);
  }
  auto snapshot = [&]() -> UnitMeta {
    UnitMeta m;
    int f = 0;
    if (cur >= 0) {
      f = kValid;
      if (wj == 0) f |= kSegStart | kFirst;
      if (wj == wnb - 1) f |= kSegEnd | kLast;
      if (wu == cbeg) f |= kAtStart | kFirst;
      if (wu == cend - 1) f |= kLast;
    }
    const int rem = min(kBlockTokens, wL - wj * kBlockTokens);
    m.bf = uni(wb | f << 16 | (rem > 0 ? rem : 0) << 24);
    m.j = uni(wj);
    m.hc = uni(whg | (cur >= 0 ? cur : 0) << 12);
    return m;
  };
  auto advance = [&]() {
    if (cur < 0) return;
    if (++wu == cend) {
      next_chunk();
      return;
    }
    if (++wj < wnb) return;
    wj = 0;
    if (++whg < HGC) return;
    whg = 0;
    do {                  // wu < cend guarantees a non-empty sequence follows
      ++wb;
      wL = uni(s_lens[wb]);
      wnb = nblocks(wL);
    } while (wnb == 0 && wb + 1 < B);
  };

  const uint32_t tok_stride = (uint32_t)Hkv * ROWB;       // bytes between tokens of a block
  const uint32_t blk_stride = kBlockTokens * tok_stride;  // bytes between physical blocks
  const uint8_t* const kpool = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* const vpool = static_cast<const uint8_t*>(a.v_pool);
  const uint8_t* const qbase = static_cast<const uint8_t*>(a.q);
  // per-lane byte offsets inside one kv head's slice of a block (constant)
  const uint32_t koff = (lane & 15) * tok_stride + (lane >> 4) * 16;
  // KLDS: load s of a block takes token rows TPI*s .. TPI*s + TPI - 1 whole (LPT lanes per
  // row); lane l writes LDS row l / LPT, slot l % LPT, and so fetches the 16-byte chunk the
  // swizzle (chunk ^ (row mod LPT)) stores there
  constexpr int LPT = ROWB / 16 < kWave ? ROWB / 16 : kWave;   // lanes per K token row
  constexpr int TPI = kWave / LPT;                             // token rows per load
  const uint32_t kdma_off = (uint32_t)(lane / LPT) * tok_stride +
                            (uint32_t)((lane % LPT) ^ ((lane / LPT) & (LPT - 1))) * 16u;
  auto kslot = [&](int u) -> uint8_t* {
    return (u == 0 ? s_kr0 : (u == 1 ? s_kr1 : (u == 2 ? s_kr2 : s_kr3))) + wave * KBLK;
  };
  // KLDS: the K operand of the unit in ring slot u, back from LDS in the layout of the
  // matrix-core loads (lane (t, q) = (lane % 16, lane / 16): chunk 4s + q of token t)
  auto kload = [&](u32x4(&kc)[NL], int u) {
    const int t = lane & 15;
    const uint8_t* kr = kslot(u) + t * ROWB;
#pragma unroll
    for (int s = 0; s < NL; ++s)
      kc[s] = *reinterpret_cast<const u32x4*>(kr + (((4 * s + (lane >> 4)) ^ (t & (LPT - 1))) * 16));
  };
  const uint32_t voff = MPV ? (4 * (lane >> 4)) * tok_stride + (lane & 15) * VB
                            : (lane / LPR) * tok_stride + (lane % LPR) * VB;
  const uint32_t vstep = MPV ? tok_stride : RPI * tok_stride;   // between a lane's V loads

  // physical id of a unit's block (every lane reads the same word); zero-size descriptor
  // for units past the range, so the load costs nothing
  auto load_id = [&](const UnitMeta& m) -> uint32_t {
    const bool v = m.flags() & kValid;
    const int32_t* row = a.block_tables + (size_t)(v ? m.b() : 0) * a.max_blocks_per_seq;
    return buf_load4(make_rsrc(row, v ? (uint32_t)a.max_blocks_per_seq * 4u : 0u),
                     (uint32_t)m.j * 4u);
  };
  // K, V of the unit's block for this wave's kv head, and the head's q rows when the
  // unit opens a piece. Always the same instructions, so wait counts stay static.
  // A block id outside [0, num_blocks) is never dereferenced: its unit keeps rem = 0, so
  // all 16 of its tokens are masked out of the softmax like rows past L.
  auto issue = [&](auto pol, UnitMeta& m, uint32_t idv, u32x4(&kb)[NL], VT(&vb)[NLV],
                   u32x4(&qs)[QPL], int slot) {
    constexpr int POL = decltype(pol)::value;
    const int pid = __builtin_amdgcn_readfirstlane((int)idv);
    const bool valid = (m.flags() & kValid) && (unsigned)pid < (unsigned)a.num_blocks;
    if (!valid) m.bf &= 0x00ffffff;
    const int g = m.hg() * NW + wave;
    const size_t base = valid ? (size_t)pid * blk_stride + (size_t)g * ROWB : 0;
    // rows at or past L (the block's last rem tokens are valid) read as zero, unfetched
    const uint32_t bytes = valid ? (uint32_t)(m.rem() - 1) * tok_stride + ROWB : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vpool + base, bytes);
    const bool wantq = (m.flags() & (kValid | kFirst)) == (kValid | kFirst);
    const size_t qo = wantq ? ((size_t)m.b() * Hq + (size_t)g * G) * D * QB : 0;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qbase + qo, wantq ? (uint32_t)QBYTES : 0u);
#pragma unroll
    for (int i = 0; i < QPL; ++i) qs[i] = buf_load16(rq, (uint32_t)(lane + kWave * i) * 16u);
    // K and V with the workgroup's cache policy (streaming unless blocks are shared)
    if constexpr (KLDS) {
      static_assert(TPI * NL == kBlockTokens && NBUF + 1 <= 4, "K ring in LDS");
#pragma unroll
      for (int s = 0; s < NL; ++s)
        buf_load16_lds(rk, kslot(slot) + s * TPI * ROWB, kdma_off + (uint32_t)(s * TPI) * tok_stride);
    } else {
#pragma unroll
      for (int s = 0; s < NL; ++s) kb[s] = buf_load16<POL>(rk, koff + s * 64);
    }
#pragma unroll
    for (int i = 0; i < NLV; ++i) vb[i] = VChunk<VB>::template load<POL>(rv, voff + i * vstep);
  };

  // ---- 4. running state of the current piece
  u32x4 qreg[NL][QCH];
  float m[HPL], lsum[HPL];                 // vector-ALU path: per head of the lane's rows
  float acc[G][VEPC];                      // vector-ALU P.V: lane (r, c), all G heads
  float m1 = 0.0f, l1 = 0.0f;              // matrix-core path: head n % G, partial l
  float qks = a.qk_scale_log2;             // score scale of the piece's kv head (log2 units)
  // matrix-core path: the softmax takes the max of the raw scores and folds the scale into
  // the exponent's fma, which needs a scale >= 0; a negative one is moved onto q (an exact
  // sign flip of its 16-bit elements). At least the smallest normal float, so that a
  // masked score of -inf times it stays -inf (finite scores times it round to equal
  // weights, as with a zero scale).
  float qka = 0.0f;
  f32x4 acc4[DPL];                         // matrix-core P.V: dim DPL*n + e, rows 4kq + v
  bool piece_whole_start = false;          // the current piece began at its segment's start
  int piece_slot = 0;
  float* const pw = &s_p[wave][0];
  uint8_t* const qw = &s_q[wave][0];

  auto compute = [&](const UnitMeta& mu, const u32x4(&kb)[NL], const VT(&vb)[NLV],
                     const u32x4(&qs)[QPL], float* P) {
    const int fl = mu.flags();
    if (!(fl & kValid)) return;
    const int g = mu.hg() * NW + wave;
    if (fl & kFirst) {
      // a new piece: fresh (m, l, acc), and this head's q rows into the MFMA operand layout
      if constexpr (MPV) {
        m1 = neg_inf();
        l1 = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc4[e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      } else {
#pragma unroll
        for (int r = 0; r < HPL; ++r) {
          m[r] = neg_inf();
          lsum[r] = 0.0f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEPC; ++e) acc[h][e] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < QPL; ++i)
        if ((lane + kWave * i) * 16 < QBYTES)
          *reinterpret_cast<u32x4*>(qw + (lane + kWave * i) * 16) = qs[i];
      wave_lds_sync();
      const uint8_t* qrow = qw + ((lane & 15) % G) * D * QB;
#pragma unroll
      for (int s = 0; s < NL; ++s) {
        const int c = 4 * s + (lane >> 4);
#pragma unroll
        for (int u = 0; u < QCH; ++u)
          qreg[s][u] = *reinterpret_cast<const u32x4*>(qrow + c * EPC * QB + u * 16);
      }
      piece_whole_start = (fl & kSegStart) != 0;
      piece_slot = (fl & kAtStart) ? 0 : 1;
      // per-head dequantisation: kv head g's K codes times k_head_scales[g]
      if constexpr (PH) qks = (a.qk_scale * a.k_head_scales[g]) * kLog2e;
      if constexpr (MPV) {
        static_assert(QB == 2, "16-bit q on the matrix-core path");
        qka = fmaxf(fabsf(qks), __FLT_MIN__);
        if (qks < 0.0f) {
#pragma unroll
          for (int s2 = 0; s2 < NL; ++s2)
#pragma unroll
            for (int u = 0; u < QCH; ++u) qreg[s2][u] ^= 0x80008000u;
        }
      }
    }
    const int rem = mu.rem();              // tokens of this block below L
    const bool ragged = rem < kBlockTokens;
    if constexpr (MPV) {
      // lane (n, kq): scores of tokens 4kq + v (v < 4) for head n % G
      const int kq = lane >> 4;
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NL; ++s) sc = kq_chunk<KV>(sc, kb[s], qreg[s]);
      // raw scores (tokens at or past L: -inf); the max commutes with the non-negative
      // scale, rounding included
      float sv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) sv[v] = sc[v];
      // only a sequence's last block is ragged: a branch on the (uniform) flag, kept as one
      // by the empty asm, which the compiler cannot turn into selects run on every unit
      if (ragged) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sv[v] = 4 * kq + v < rem ? sv[v] : neg_inf();
          asm volatile("" : "+v"(sv[v]));
        }
      }
      // new running max of head n % G: over the lane's 4 tokens and the running max, then
      // over the 4 row groups, which hold the block's other tokens
      const float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])) * qka;
      const float mn = xrow_max(fmaxf(bm, m1));
      const float al1 = mn == neg_inf() ? 1.0f : fast_exp2(m1 - mn);
      // (mn is -inf only while every token so far was masked: then every p is 0)
      const float mref = mn == neg_inf() ? 0.0f : mn;
      float pf[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) pf[v] = fast_exp2(fmaf(sv[v], qka, -mref));   // 0 if masked
      // the matrix cores take p in 16 bits, as a hi and a lo part (within 2^-16 of p)
      const u32x4 aop = split_pack4<KV>(pf);
      l1 = l1 * al1 + ((pf[0] + pf[1]) + (pf[2] + pf[3]));
      m1 = mn;
      // rescale: accumulator row 4kq + v belongs to head (4kq + v) % G, whose factor lives
      // in the lanes of column n with n % G == that head
      if (__builtin_amdgcn_ballot_w64(al1 != 1.0f) != 0) {
        float alv[4];
        if constexpr (G <= 4) {
          alv[0] = quad_bcast<0>(al1);
          alv[1] = quad_bcast<1 % G>(al1);
          alv[2] = quad_bcast<2 % G>(al1);
          alv[3] = quad_bcast<3 % G>(al1);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) alv[v] = __shfl(al1, (lane & 48) + 4 * (kq & 1) + v);
        }
#pragma unroll
        for (int e = 0; e < DPL; ++e)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc4[e][v] *= alv[v];
      }
      // B operands: token rows 4kq + i of this lane's dims (rows at or past L read as zero)
      if constexpr (KV == PA_FP8_E4M3) {
        // fp8: interleave the bytes of tokens 2p and 2p + 1 first (one byte permute per two
        // dims), so that each conversion yields the bf16 pair (token 2p, token 2p + 1) of
        // one dim, which is a half of the B operand as it is
        uint32_t pw[2][DPL];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
#pragma unroll
          for (int w = 0; w < DPL / 4; ++w) {
            const uint32_t a = vb[2 * pr][w], b = vb[2 * pr + 1][w];
            const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
            const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
            pw[pr][4 * w] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
            pw[pr][4 * w + 1] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
            pw[pr][4 * w + 2] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
            pw[pr][4 * w + 3] = __builtin_bit_cast(
                uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
          }
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc4[e] = mfma_pv<KV>(aop, u32x2{pw[0][e], pw[1][e]}, acc4[e]);
      } else {
        constexpr int WORDS = DPL / 2;
        uint32_t vw[4][WORDS];
#pragma unroll
        for (int i = 0; i < 4; ++i) v_words16<KV, WORDS>(vb[i], vw[i]);
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const u32x2 bop = {__builtin_amdgcn_perm(vw[1][e >> 1], vw[0][e >> 1], sel),
                             __builtin_amdgcn_perm(vw[3][e >> 1], vw[2][e >> 1], sel)};
          acc4[e] = mfma_pv<KV>(aop, bop, acc4[e]);
        }
      }
    } else {
      // vector-ALU P.V (fp32 K/V). Scores of token t = lane % 16 for the heads of MFMA rows
      // 4*(lane/16) + r.
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NL; ++s) sc = qk_chunk_f32(sc, kb[s], qreg[s]);
      const bool tok_ok = (lane & 15) < rem;
      // (tok_ok holds on every lane of a full block, so the masks need no branch)
      float al[HPL], p[HPL], sv[HPL], mn[HPL];
#pragma unroll
      for (int r = 0; r < HPL; ++r) {
        sv[r] = tok_ok ? sc[r] * qks : neg_inf();
        mn[r] = sv[r] > m[r] ? sv[r] : m[r];   // m is the same on all lanes of a row
      }
      row16_max_n<HPL>(mn);                  // new running maxima, one per head
#pragma unroll
      for (int r = 0; r < HPL; ++r) {
        al[r] = mn[r] == neg_inf() ? 1.0f : fast_exp2(m[r] - mn[r]);
        p[r] = tok_ok ? fast_exp2(sv[r] - mn[r]) : 0.0f;
        lsum[r] = lsum[r] * al[r] + p[r];
        m[r] = mn[r];
      }
      if ((lane >> 4) < QROWS) {
        const int hb = G > 4 ? 4 * (lane >> 4) : 0;
        float* dst = P + (lane & 15) * G + hb;
#pragma unroll
        for (int r = 0; r < HPL; ++r) dst[r] = p[r];
        if constexpr (G > 4) {
          if ((lane & 15) == 0)
#pragma unroll
            for (int r = 0; r < HPL; ++r) P[kBlockTokens * G + hb + r] = al[r];
        }
      }
      wave_lds_sync();
      float alpha[G];
      if constexpr (G > 4) {
#pragma unroll
        for (int h = 0; h < G; ++h) alpha[h] = P[kBlockTokens * G + h];
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) alpha[h] = al[h];
      }
      bool moved = false;
#pragma unroll
      for (int h = 0; h < G; ++h) moved |= alpha[h] != 1.0f;
      if (moved) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEPC; ++e) acc[h][e] *= alpha[h];
      }
      // V rows at or past L read as zero
#pragma unroll
      for (int i = 0; i < NLV; ++i) {
        const int row = lane / LPR + RPI * i;
        float pv[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pv[h] = P[row * G + h];
        float v[VEPC];
#pragma unroll
        for (int e = 0; e < VEPC; ++e) v[e] = __uint_as_float(vb[i][e]);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEPC; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
      }
    }

    if (!(fl & kLast)) return;
    // ---- the piece ends here: reduce over lanes, then write the output (whole segment)
    // or a record (a piece of a segment cut by a chunk boundary)
    const bool whole = piece_whole_start && (fl & kSegEnd);
    const float vsc = PH ? a.v_head_scales[g] : a.v_scale;
    const size_t rec = ((size_t)mu.chunk() * 2 + piece_slot) * NW + wave;
    if constexpr (MPV) {
      // l of head n % G over the whole block (the row groups held partial sums); lanes of
      // row group kq < QROWS write heads hb + v (v < HPL) for dims DPL*n + e, taking m and
      // l of head h from lane h
      const float lt = xrow_sum(l1);
      float m[HPL], lsum[HPL];
      const int hb = G > 4 ? 4 * (lane >> 4) : 0;
#pragma unroll
      for (int v = 0; v < HPL; ++v) {
        m[v] = __shfl(m1, (hb + v) & 15);
        lsum[v] = __shfl(lt, (hb + v) & 15);
      }
      if ((lane >> 4) < QROWS) {
        const int n = lane & 15;
#pragma unroll
        for (int v = 0; v < HPL; ++v) {
          const int h = hb + v;
          if (whole) {
            const size_t o = ((size_t)mu.b() * Hq + (size_t)g * G + h) * D + DPL * n;
            const float inv = lsum[v] > 0.0f ? vsc / lsum[v] : 0.0f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) store_out<OT>(a.out, o + e, acc4[e][v] * inv);
          } else {
#pragma unroll
            for (int e = 0; e < DPL; ++e)
              a.rec_acc[(rec * G + h) * D + DPL * n + e] = acc4[e][v];
            if (n == 0) {
              a.rec_ml[(rec * G + h) * 2] = m[v];
              a.rec_ml[(rec * G + h) * 2 + 1] = lsum[v];
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < HPL; ++r) lsum[r] = row16_sum(lsum[r]);
#pragma unroll
      for (int st = LPR; st < kWave; st <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < VEPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], st);
      float mh[G], lh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if constexpr (G > 4) {
          mh[h] = __shfl(m[h & 3], (h >> 2) * 16);
          lh[h] = __shfl(lsum[h & 3], (h >> 2) * 16);
        } else {
          mh[h] = m[h];
          lh[h] = lsum[h];
        }
      }
      if (whole) {
        if (lane < LPR) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const size_t o = ((size_t)mu.b() * Hq + (size_t)g * G + h) * D + VEPC * lane;
            const float inv = lh[h] > 0.0f ? vsc / lh[h] : 0.0f;
#pragma unroll
            for (int e = 0; e < VEPC; ++e) store_out<OT>(a.out, o + e, acc[h][e] * inv);
          }
        }
      } else {
        if (lane < LPR) {
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < VEPC; ++e)
              a.rec_acc[(rec * G + h) * D + VEPC * lane + e] = acc[h][e];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (lane == h) {
            a.rec_ml[(rec * G + h) * 2] = mh[h];
            a.rec_ml[(rec * G + h) * 2 + 1] = lh[h];
          }
        }
      }
    }
  };

  // ---- 5. the stream, over a ring of R = NBUF + 1 register slots (unit x lives in slot
  // x % R). Step k first issues the K/V loads of unit k + NBUF into the slot unit k - 1
  // has just left (its block id was loaded R steps earlier) and the id load of unit
  // k + NBUF + R, then computes unit k: NBUF units stay in flight while one is computed.
  // The ring is unrolled so that every slot index is a constant. It is compiled once per
  // cache policy of the K/V loads.
  constexpr int R = NBUF + 1;
  auto stream = [&](auto pol) {
    u32x4 kb[R][NL];
    VT vb[R][NLV];
    u32x4 qs[R][QPL];
    uint32_t idv[R];
    UnitMeta mk[R], mi[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      mi[u] = snapshot();
      idv[u] = load_id(mi[u]);
      advance();
    }
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      mk[u] = mi[u];
      issue(pol, mk[u], idv[u], kb[u], vb[u], qs[u], u);
      mi[u] = snapshot();
      idv[u] = load_id(mi[u]);
      advance();
    }
    u32x4 kcur[NL];
    if constexpr (KLDS) kload(kcur, 0);
    if (!cg.fixed && wave == 0 && lane == 0) {
      int4 hd = make_int4(-1, 0, 0, 0);
      if (hdr_b >= 0) {
        const int cf = chunk_of(cg, hdr_sseg);
        hd = make_int4(hdr_b, hdr_hg, cf, chunk_begin(cg, cf) < hdr_sseg ? 1 : 0);
      }
      *reinterpret_cast<int4*>(a.chunk_hdr + 4 * hdr_c) = hd;
    }
    // every wave sees the same chunks, so the loop ends at the same step in all of them
    for (;;) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int si = (u + NBUF) % R;   // slot of unit k + NBUF (= slot of unit k - 1)
        mk[si] = mi[si];
        issue(pol, mk[si], idv[si], kb[si], vb[si], qs[si], si);
        mi[si] = snapshot();
        idv[si] = load_id(mi[si]);
        advance();
        if constexpr (KLDS) {
          // K of unit k came back from LDS during step k - 1; unit k + 1's is read now,
          // after unit k's matrix-core work is issued
          compute(mk[u], kcur, vb[u], qs[u], pw + (u & 1) * PBUF);
          kload(kcur, (u + 1) % R);
        } else {
          compute(mk[u], kb[u], vb[u], qs[u], pw + (u & 1) * PBUF);
        }
      }
      bool busy = cur >= 0;
#pragma unroll
      for (int u = 0; u < R; ++u) busy |= ((mk[u].flags() | mi[u].flags()) & kValid) != 0;
      if (!busy) break;
    }
  };
  if (wg_shared)
    stream(std::integral_constant<int, kCached>{});
  else
    stream(std::integral_constant<int, kStream>{});
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int st = 1; st < kWave; st <<= 1) x += __shfl_xor(x, st);
  return x;
}

// N consecutive floats from an address aligned to the widest of 16, 8 or 4 bytes that N
// floats fill, as vector loads.
template <int N>
__device__ __forceinline__ void load_floats(const float* p, float (&x)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 v = reinterpret_cast<const f32x4*>(p)[i];
      x[4 * i] = v[0];
      x[4 * i + 1] = v[1];
      x[4 * i + 2] = v[2];
      x[4 * i + 3] = v[3];
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const f32x2 v = reinterpret_cast<const f32x2*>(p)[i];
      x[2 * i] = v[0];
      x[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
  }
}

// Fixed partitions, and the default split when a call can have few units per chunk (so
// that a segment may be cut into many pieces): combine the pieces of segments cut by
// chunk boundaries, with the same rescaling: M = max_p m_p,
// out = v_scale * sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), with v_scale the
// per-tensor scale or kv head g's own.
// Also writes zeros for sequences of length 0 (they own no units). One workgroup of MW
// waves per (kv head, sequence, one of NS slices of the head dimension): a few long sequences
// still spread the merge over many CUs. Lane i of a wave handles EPL consecutive outputs
// of query head h within the slice. Wave w folds pieces w, w + MW, ... into a running
// (M, L, A) with the online rule, UNROLL pieces per memory round trip (more when a lane
// holds fewer outputs: all of a 32k-token sequence's 256 one-block pieces in one trip
// with NS = 8); the MW partial results are then combined through LDS.
// waves of a fixed-partition merge workgroup: 16, or 8 when a slice's G * D / NS outputs
// are 1024 (the partial results then still fit 32 KB of LDS)
template <int G, int D, int NS>
constexpr int merge_waves() { return G * D / NS >= 1024 ? 8 : 16; }

template <int OT, int D, int G, int NS>
__global__ __launch_bounds__(1024) void merge_kernel(MergeArgs a) {
  constexpr int DS = D / NS;               // dims of the slice
  constexpr int EPL = G * DS / kWave;
  constexpr int MWMAX = merge_waves<G, D, NS>();
  constexpr int UNROLL = EPL >= 8 ? 4 : (EPL >= 4 ? 8 : 16);   // as the host assumes
  static_assert(EPL >= 1 && DS % EPL == 0, "merge layout");
  __shared__ float s_ml[MWMAX][G][2];
  __shared__ float s_acc[MWMAX][G * DS];
  const int MW = blockDim.x / kWave;       // 4 .. MWMAX, from the pieces a segment typically has
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int g = blockIdx.x / NS, b = blockIdx.y;
  const int h = lane * EPL / DS, d0 = (int)(blockIdx.x % NS) * DS + (lane * EPL) % DS;
  const int dl = (lane * EPL) % DS;        // position within the slice
  const size_t o = ((size_t)b * a.num_q_heads + (size_t)g * G + h) * D + d0;
  const int c0 = a.prefix[b], nb = a.prefix[b + 1] - c0, total = a.prefix[a.batch];
  if (nb == 0) {
    if (wave == 0)
#pragma unroll
      for (int i = 0; i < EPL; ++i) store_out<OT>(a.out, o + i, 0.0f);
    return;
  }
  const int NW = a.group_waves, HGC = a.num_kv_heads / NW;
  const int hg = g / NW, wv = g % NW;
  const int64_t T = (int64_t)HGC * total;
  const int64_t S = (int64_t)HGC * c0 + (int64_t)hg * nb, E = S + nb - 1;
  const ChunkGeom cg = chunk_geometry(T, a.num_ranges, a.part_units);
  const int W = cg.W;
  // The segment's pieces, in unit order: the chunks it overlaps, which hold at most one
  // unit each when T < W (then a piece per unit, in chunk ((u + 1) W - 1) / T, so the
  // empty chunks between them are never visited; 32-bit: u < T < W <= kMaxChunks).
  const bool by_unit = T < W;
  const int Ti = (int)T, Si = (int)S, Ei = (int)E;
  int cf, np;
  if (by_unit) {
    cf = ((Si + 1) * W - 1) / Ti;
    np = Ei - Si + 1;
  } else {
    cf = chunk_of(cg, S);
    np = chunk_of(cg, E) - cf + 1;
  }
  if (np == 1) return;                   // one chunk held the whole segment
  // records of chunk c: its first piece is in slot 0, its last (if different) in slot
  // 1; only chunk cf can hold the segment as its last piece
  const int slot_f = chunk_begin(cg, cf) < S ? 1 : 0;
  auto rec_of = [&](int c, int k) -> size_t {   // piece k of the segment, in chunk c
    return (((size_t)c * 2 + (k == 0 ? slot_f : 0)) * NW + wv) * G + h;
  };

  float M = neg_inf(), L = 0.0f, A[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) A[i] = 0.0f;
  for (int kb = wave; kb < np; kb += MW * UNROLL) {
    // the round's loads are issued together and stop at the last piece. One unit per
    // chunk: lane u works out the chunk of piece kb + u MW, so the round's divisions run
    // side by side, and each load reads its chunk from that lane.
    int cl = 0;
    if (by_unit) {
      const int kk = kb + (lane % UNROLL) * MW;
      cl = ((Si + (kk < np ? kk : 0) + 1) * W - 1) / Ti;
    }
    f32x2 mlp[UNROLL];
    float x[UNROLL][EPL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = kb + u * MW;
      if (k >= np) break;   // (the same in the whole wave)
      const size_t rec = rec_of(by_unit ? __builtin_amdgcn_readlane(cl, u) : cf + k, k);
      mlp[u] = *reinterpret_cast<const f32x2*>(a.rec_ml + rec * 2);
      load_floats<EPL>(a.rec_acc + rec * D + d0, x[u]);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (kb + u * MW >= np) continue;
      const float Mn = fmaxf(M, mlp[u].x);
      if (Mn == neg_inf()) continue;     // nothing yet
      const float sa = M == neg_inf() ? 0.0f : fast_exp2(M - Mn);
      const float sb = mlp[u].x == neg_inf() ? 0.0f : fast_exp2(mlp[u].x - Mn);
      L = L * sa + mlp[u].y * sb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) A[e] = A[e] * sa + x[u][e] * sb;
      M = Mn;
    }
  }
  if (dl == 0) {
    s_ml[wave][h][0] = M;
    s_ml[wave][h][1] = L;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][h * DS + dl + e] = A[e];
  __syncthreads();
  if (wave != 0) return;
  float Mt = neg_inf();
#pragma unroll
  for (int w = 0; w < MW; ++w) Mt = fmaxf(Mt, s_ml[w][h][0]);
  float Lt = 0.0f, At[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) At[e] = 0.0f;
#pragma unroll 2
  for (int w = 0; w < MW; ++w) {
    const float mw = s_ml[w][h][0];
    const float f = mw == neg_inf() ? 0.0f : fast_exp2(mw - Mt);
    Lt = fmaf(s_ml[w][h][1], f, Lt);
#pragma unroll
    for (int e = 0; e < EPL; ++e) At[e] = fmaf(s_acc[w][h * DS + dl + e], f, At[e]);
  }
  const float vsc = a.v_head_scales ? a.v_head_scales[g] : a.v_scale;
  const float inv = Lt > 0.0f ? vsc / Lt : 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) store_out<OT>(a.out, o + i, At[i] * inv);
}

// Default split: combine the pieces of the segment whose last piece opens chunk c, as
// named by chunk c's header, with the same rescaling (v_scale per tensor or per kv head).
// Wave w handles kv head hg * NW + w; lane i holds EPL consecutive outputs of query head
// h. The header, chunk c's first record and chunk c - 1's last record are loaded
// together, so a segment cut once (nearly all of them) costs one memory round trip;
// a segment spread over more chunks loads its other pieces UNROLL at a time.
template <int OT, int D, int G>
__global__ __launch_bounds__(kMaxThreads) void merge_chunk_kernel(MergeArgs a) {
  constexpr int EPL = G * D / kWave;
  constexpr int UNROLL = 8;
  static_assert(EPL >= 1 && D % EPL == 0, "merge layout");
  // chunk c is merged on the XCD whose workgroup decoded it (the decode's dealing of
  // chunks to workgroup ids), where its records and their address translations are
  // still cached
  const int W = a.num_ranges, bid = blockIdx.x;
  const int c = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int NW = a.group_waves;
  const int h = lane * EPL / D, d0 = (lane * EPL) % D;
  auto rec_of = [&](int chunk, int slot) -> size_t {
    return (((size_t)chunk * 2 + slot) * NW + wave) * G + h;
  };
  const int4 hd = *reinterpret_cast<const int4*>(a.chunk_hdr + 4 * c);
  const int total = a.prefix[a.batch];    // needed only by segments over 3+ chunks
  const size_t r1 = rec_of(c, 0), r0 = rec_of(c > 0 ? c - 1 : 0, 1);
  const f32x2 ml1 = *reinterpret_cast<const f32x2*>(a.rec_ml + r1 * 2);
  const f32x2 ml0 = *reinterpret_cast<const f32x2*>(a.rec_ml + r0 * 2);
  float x1[EPL], x0[EPL];
  load_floats<EPL>(a.rec_acc + r1 * D + d0, x1);
  load_floats<EPL>(a.rec_acc + r0 * D + d0, x0);
  // keep the record loads ahead of the header test (otherwise they are sunk below it
  // and cost a second round trip)
  asm volatile("" ::"v"(ml1.x), "v"(ml1.y), "v"(ml0.x), "v"(ml0.y), "s"(total));
#pragma unroll
  for (int e = 0; e < EPL; ++e) asm volatile("" ::"v"(x1[e]), "v"(x0[e]));
  const int b = hd.x;
  if (b < 0) return;
  const int hg = hd.y, cf = hd.z, slot_f = hd.w;

  float M = neg_inf(), L = 0.0f, A[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[e] = 0.0f;
  auto fold = [&](float mp, float lp, const float* x) {
    const float Mn = fmaxf(M, mp);
    if (Mn == neg_inf()) return;         // nothing yet
    const float sa = M == neg_inf() ? 0.0f : fast_exp2(M - Mn);
    const float sb = mp == neg_inf() ? 0.0f : fast_exp2(mp - Mn);
    L = L * sa + lp * sb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) A[e] = A[e] * sa + x[e] * sb;
    M = Mn;
  };
  if (cf == c - 1 && slot_f == 1) {
    fold(ml0.x, ml0.y, x0);
  } else {
    // pieces in chunks cf .. c-1 (slot slot_f in chunk cf, else 0). Static chunks are
    // empty only when there are fewer units than chunks (T < W); each then holds at most
    // one unit, so the pieces are the segment's units before chunk c's, unit u in chunk
    // ((u + 1) W - 1) / T (32-bit: T < W <= 2048).
    const int64_t T = (int64_t)(a.num_kv_heads / NW) * total;
    const int Ts = T < W ? (int)T : 0;
    const int u0 = Ts > 0 ? Ts * cf / W : 0;             // the segment's first unit
    const int n = Ts > 0 ? Ts * c / W - u0 : c - cf;     // pieces before chunk c
    for (int kb = 0; kb < n; kb += UNROLL) {
      // the round's loads are issued together (one round trip for up to UNROLL pieces)
      // and stop at the last piece. One unit per chunk: lane u works out the chunk of
      // piece kb + u (divisions side by side).
      int cl = c;
      if (Ts > 0) {
        const int kk = kb + lane % UNROLL;
        cl = kk >= n ? c : ((u0 + kk + 1) * W - 1) / Ts;
      }
      f32x2 mlp[UNROLL];
      float x[UNROLL][EPL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int k = kb + u;
        if (k >= n) break;   // (the same in the whole wave)
        const int cc = Ts > 0 ? __builtin_amdgcn_readlane(cl, u) : cf + k;
        const size_t rec = rec_of(cc, (k == 0) ? slot_f : 0);
        mlp[u] = *reinterpret_cast<const f32x2*>(a.rec_ml + rec * 2);
        load_floats<EPL>(a.rec_acc + rec * D + d0, x[u]);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        if (kb + u < n) fold(mlp[u].x, mlp[u].y, x[u]);
    }
  }
  fold(ml1.x, ml1.y, x1);
  const int g = hg * NW + wave;
  const float vsc = a.v_head_scales ? a.v_head_scales[g] : a.v_scale;
  const float inv = L > 0.0f ? vsc / L : 0.0f;
  const size_t o = ((size_t)b * a.num_q_heads + (size_t)g * G + h) * D + d0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) store_out<OT>(a.out, o + e, A[e] * inv);
}

template <int KV, int QT, int OT, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& args, int nw, hipStream_t stream) {
  const dim3 grid(args.num_ranges), block(nw * kWave);
  if constexpr (KV == PA_FP8_E4M3) {
    if (args.k_head_scales) {
      decode_kernel<KV, QT, OT, D, G, true><<<grid, block, 0, stream>>>(args);
      return hipGetLastError();
    }
  }
  decode_kernel<KV, QT, OT, D, G, false><<<grid, block, 0, stream>>>(args);
  return hipGetLastError();
}

template <int KV, int QT, int OT, int D>
hipError_t dispatch_group(int group, const DecodeArgs& args, int nw, hipStream_t stream) {
  switch (group) {
    case 1: return launch_decode_t<KV, QT, OT, D, 1>(args, nw, stream);
    case 2: return launch_decode_t<KV, QT, OT, D, 2>(args, nw, stream);
    case 4: return launch_decode_t<KV, QT, OT, D, 4>(args, nw, stream);
    case 8: return launch_decode_t<KV, QT, OT, D, 8>(args, nw, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, int QT, int OT>
hipError_t dispatch_dim(int head_dim, int group, const DecodeArgs& args, int nw,
                        hipStream_t stream) {
  switch (head_dim) {
    case 64: return dispatch_group<KV, QT, OT, 64>(group, args, nw, stream);
    case 128: return dispatch_group<KV, QT, OT, 128>(group, args, nw, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int OT, int D>
hipError_t launch_merge_t(int group, const MergeArgs& args, hipStream_t stream) {
  if (args.part_units == 0 && args.chunk_merge) {   // one workgroup per chunk
    const dim3 grid(args.num_ranges), block(args.group_waves * kWave);
    switch (group) {
      case 1: merge_chunk_kernel<OT, D, 1><<<grid, block, 0, stream>>>(args); break;
      case 2: merge_chunk_kernel<OT, D, 2><<<grid, block, 0, stream>>>(args); break;
      case 4: merge_chunk_kernel<OT, D, 4><<<grid, block, 0, stream>>>(args); break;
      case 8: merge_chunk_kernel<OT, D, 8><<<grid, block, 0, stream>>>(args); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // 4 waves fold 16 or more pieces per round trip; more waves only when a segment can
  // have more pieces (most workgroups of a large batch exit at once, and launching idle
  // waves costs). Slices of the head dimension when there are few (kv head, sequence)
  // pairs, up to 8 and while a lane keeps at least one output.
  int S = 1;
  while (S < 8 && (int64_t)args.num_kv_heads * args.batch * S < 512 && group * D >= 128 * S)
    S *= 2;
  const dim3 grid(args.num_kv_heads * S, args.batch);
  auto launch = [&](auto g_tag, auto s_tag) {
    constexpr int GG = decltype(g_tag)::value, SS = decltype(s_tag)::value;
    if constexpr (GG * D >= 64 * SS) {
      // enough waves for the pieces a segment typically has in one round trip, and at
      // least 4, so that the folds of a few pieces run side by side
      constexpr int EPL = GG * D / SS / kWave, UN = EPL >= 8 ? 4 : (EPL >= 4 ? 8 : 16);
      const int need = (args.max_pieces + UN - 1) / UN;
      int waves = 4;
      while (waves < need && waves < merge_waves<GG, D, SS>()) waves *= 2;
      merge_kernel<OT, D, GG, SS><<<grid, waves * kWave, 0, stream>>>(args);
    }
  };
  auto by_slices = [&](auto g_tag) {
    switch (S) {
      case 1: launch(g_tag, std::integral_constant<int, 1>{}); break;
      case 2: launch(g_tag, std::integral_constant<int, 2>{}); break;
      case 4: launch(g_tag, std::integral_constant<int, 4>{}); break;
      default: launch(g_tag, std::integral_constant<int, 8>{}); break;
    }
  };
  switch (group) {
    case 1: by_slices(std::integral_constant<int, 1>{}); break;
    case 2: by_slices(std::integral_constant<int, 2>{}); break;
    case 4: by_slices(std::integral_constant<int, 4>{}); break;
    case 8: by_slices(std::integral_constant<int, 8>{}); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                         const DecodeArgs& args, int nw, hipStream_t stream) {
  if (q_dtype == PA_F32 && kv_dtype == PA_F32 && out_dtype == PA_F32)
    return dispatch_dim<PA_F32, PA_F32, PA_F32>(head_dim, group, args, nw, stream);
  if (q_dtype == PA_F16 && kv_dtype == PA_F16) {
    if (out_dtype == PA_F16)
      return dispatch_dim<PA_F16, PA_F16, PA_F16>(head_dim, group, args, nw, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_F16, PA_F16, PA_F32>(head_dim, group, args, nw, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_BF16) {
    if (out_dtype == PA_BF16)
      return dispatch_dim<PA_BF16, PA_BF16, PA_BF16>(head_dim, group, args, nw, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_BF16, PA_BF16, PA_F32>(head_dim, group, args, nw, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3) {
    if (out_dtype == PA_BF16)
      return dispatch_dim<PA_FP8_E4M3, PA_BF16, PA_BF16>(head_dim, group, args, nw, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_FP8_E4M3, PA_BF16, PA_F32>(head_dim, group, args, nw, stream);
  }
  return hipErrorInvalidValue;
}

// The current device's address of `scratch`: hipGetSymbolAddress once per device, with
// that device current, kept for later calls.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_merge(int out_dtype, int head_dim, int group, const MergeArgs& args,
                        hipStream_t stream) {
  if (head_dim == 64) {
    if (out_dtype == PA_F32) return launch_merge_t<PA_F32, 64>(group, args, stream);
    if (out_dtype == PA_F16) return launch_merge_t<PA_F16, 64>(group, args, stream);
    return launch_merge_t<PA_BF16, 64>(group, args, stream);
  }
  if (out_dtype == PA_F32) return launch_merge_t<PA_F32, 128>(group, args, stream);
  if (out_dtype == PA_F16) return launch_merge_t<PA_F16, 128>(group, args, stream);
  return launch_merge_t<PA_BF16, 128>(group, args, stream);
}

}  // namespace pa
