// pa_prefill.hip - attention of several new query tokens per sequence over a block-paged
// KV cache (chunked prefill, or the tail left after a prefix-cache hit), gfx950 (CDNA4).
//
// What is computed (LLM KV cache serving-engine article, sections 3 and 4; softmax and
// block table as in vLLM-PagedAttention与连续批处理技术拆解, sections 3.1-3.3): sequence b
// holds L tokens in its paged cache, the last n of which are its new query tokens, already
// written by the slot write. Query token i sits at position L - n + i and attends over
// positions [0, L - n + i] (causal among the new tokens); a position below zero (n > L)
// attends over nothing and gives a zero row.
//
// How it maps onto CDNA4
//   * A workgroup of 4 waves owns one (sequence, kv head, tile of TQ query tokens). Its
//     rows are (token, head) pairs, row r = token r / G, head r % G, so the G query heads
//     that share a kv head share every K/V byte: each wave owns RG groups of 16 rows.
//   * K/V are staged through LDS 64 tokens (4 blocks) at a time, double-buffered: the
//     global loads of the next tile are in flight while the current one is computed. K
//     rows reach LDS in the score type (bf16 for bf16 and fp8 K, fp16 for fp16; fp8
//     widened exactly), V rows in fp16 (fp8 widened exactly, bf16 converted: see below).
//     16-bit K goes from HBM straight into LDS (buffer loads with the lds bit), requested
//     after the tile's score MFMAs, its rows unpadded with the 16-byte chunks XOR-swizzled
//     by row; fp8 K rows are padded by 16 bytes, V rows by 32, to spread the banks.
//   * The P.V operand B (eight consecutive tokens of one output dim) comes straight from
//     the row-major V tile through transposed LDS reads (ds_read_b64_tr_b16), so MFMA e
//     covers output dims 16e + n; no byte permutes.
//   * Scores run on the matrix cores as K.Q^T (v_mfma_f32_16x16x32_{bf16,f16}): lane
//     (n, kq) = (lane % 16, lane / 16) ends with the scores of tokens 4kq .. 4kq+3 of each
//     16-token subtile for row n, which is, two subtiles at a time, exactly the A-operand
//     layout P takes in P.V, so P never leaves registers.
//   * Online softmax per row (running max and normaliser l). The weights are taken
//     against a reference max that moves only when the row's max outgrows it by more than
//     2^8, so the accumulators are rescaled a few times per row instead of at most tiles
//     (exact in real arithmetic: softmax does not depend on the reference).
//     P.V runs on the matrix cores in fp16 for every K/V type: p rounded to fp16
//     (relative rounding 2^-11) against fp16 V, with the normaliser taken by the same
//     MFMAs (P times a column of ones), so that it sums exactly the rounded weights and
//     the output stays an exact weighted average of V rows. bf16 V converts to fp16
//     exactly below 2^16 in magnitude (values under 2^-17 move by less than 2^-25). Where
//     a workgroup meets a bf16 V value of 2^16 or more (or an infinity or NaN), which
//     leaves a non-finite accumulator behind, it runs its
//     key loop again with V staged as bf16 and p split into hi (p with its low 16 bits
//     cleared, exact) and lo = bf16(p - hi), both taken by bf16 MFMAs (weights exact to
//     about 2^-16, at twice the P.V matrix work). bf16 weights in one pass (rounding up
//     to 2^-9) would move the output of rows attending over a few tokens by a visible
//     fraction of the spread of V.
//   * Tiles wholly at or before the tile's first query position need no mask; the rest
//     mask positions past each row's own. A block id outside the pool is never read; its
//     16 tokens get weight 0 in every row (from the first tile holding one, every tile
//     takes the masked body).
//   * Workgroup ids are dealt so that all query tiles of one (sequence, kv head) land on
//     the same XCD (workgroups go to the 8 XCDs round-robin) and share its L2; sequences
//     go longest first, and within a pair, later tiles (longer key ranges) start first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/paged_attention.h"
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kTileTokens = 64;                      // K/V tokens per LDS tile
// LDS row padding, bytes: K rows by 16 (the 16 rows a score operand read takes then sit
// on distinct banks), V rows by 32 (the four rows a transposed read takes then do)
constexpr int kKPad = 16, kVPad = 32;
// Log2-domain growth of a row's max that moves its reference: below it, p = 2^(s - m_ref)
// may reach 2^8, which fp32 sums and the 16-bit hi/lo parts of p carry without loss, and
// the accumulators need no rescale.
constexpr float kLazyMax = 8.0f;
constexpr int kPrefillThreads = kPrefillWaves * kWave;

// One 16x16x32 MFMA in the 16-bit type CT: acc += A * B.
template <int CT>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 acc) {
  if constexpr (CT == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds): lane l
// writes lds + 16 l; a lane whose offset is out of range writes zeros.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// Two floats rounded to fp16 / bf16 (nearest even) and packed, a in the low half.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

template <int KV, int OT, int D, int G, int RG>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(PrefillArgs a) {
  constexpr int ST = KV == PA_F16 ? PA_F16 : PA_BF16;  // element type of the score MFMAs
  constexpr int KB = Enc<KV>::bytes;
  constexpr int ROWB = D * KB;                   // pool bytes of one token row, one kv head
  // 16-bit K goes from HBM straight into LDS (KDMA): rows unpadded, the 16-byte chunks of
  // row r stored at chunk ^ (r mod the chunks per row), which spreads the banks as the pad
  // does; fp8 K is widened in registers on its way and keeps the padded rows
  constexpr bool KDMA = KB == 2;
  constexpr int LROW = KDMA ? D * 2 : D * 2 + kKPad;   // LDS bytes of one K token row (16-bit)
  constexpr int VROW = D * 2 + kVPad;            // LDS bytes of one V token row (16-bit)
  constexpr int ROWS = kPrefillWaves * RG * 16;  // (token, head) rows of the workgroup
  constexpr int TQ = ROWS / G;                   // query tokens of the workgroup
  constexpr int NC = D / 32;                     // 32-dim steps of a score MFMA chain
  constexpr int DPL = D / 16;                    // output dims per lane and 16-row group
  static_assert(ROWS % G == 0 && 16 % G == 0, "rows hold whole tokens");

  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kTileTokens * LROW];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][kTileTokens * VROW];

  // ---- which (sequence, kv head, query tile): id = ((group * tiles) + tile') * 8 + x,
  // pair = group * 8 + x, tile = tiles - 1 - tile'; pair p is kv head p % Hkv of the
  // sequence ranked p / Hkv, sequences ranked longest first (ties by index) when the batch
  // has at most one sequence per thread, else in index order. Workgroups start in id order,
  // so the longest causal ranges start first and short ones fill the end of the launch.
  // (integer division runs on the vector ALU: uni() keeps the results scalar)
  const int id = blockIdx.x;
  const int x8 = id & 7, rest = id >> 3;
  const int grp = uni(rest / a.num_q_tiles);
  const int pair = grp * 8 + x8;
  if (pair >= a.batch * a.num_kv_heads) return;   // (the whole workgroup)
  const int tile = a.num_q_tiles - 1 - (rest - grp * a.num_q_tiles);
  const int rank = uni(pair / a.num_kv_heads), kvh = pair - rank * a.num_kv_heads;
  int b = rank;
  if (a.batch <= kPrefillThreads) {
    __shared__ int s_len[kPrefillThreads];
    __shared__ int s_seq;
    const int t = threadIdx.x;
    if (t < a.batch) s_len[t] = a.context_lens[t];
    __syncthreads();
    if (t < a.batch) {
      const int Lt = s_len[t];
      int r = 0;
      for (int j = 0; j < a.batch; ++j) r += s_len[j] > Lt || (s_len[j] == Lt && j < t);
      if (r == rank) s_seq = t;               // ranks are a permutation of [0, batch)
    }
    __syncthreads();
    b = uni(s_seq);
  }
  // the sequence's rows, kept inside [0, Tq) whatever query_start holds; rows past
  // max_query_len are not computed, though they still count in the positions
  const int Tq = a.num_query_tokens;
  int qs0 = a.query_start[b], qs1 = a.query_start[b + 1];
  qs0 = qs0 < 0 ? 0 : (qs0 < Tq ? qs0 : Tq);
  qs1 = qs1 < qs0 ? qs0 : (qs1 < Tq ? qs1 : Tq);
  const int n = qs1 - qs0;
  const int nr = n < a.max_query_len ? n : a.max_query_len;   // rows computed
  const int t0 = tile * TQ;
  if (t0 >= nr) return;
  const int cap = a.max_blocks_per_seq * kBlockTokens;
  int L = a.context_lens[b];
  L = L < 0 ? 0 : (L < cap ? L : cap);
  const int nb = (L + kBlockTokens - 1) / kBlockTokens;
  const int pos0 = L - n;                                  // position of query token 0
  const int last_pos = pos0 + (t0 + TQ < nr ? t0 + TQ : nr) - 1;
  const int first_pos = pos0 + t0;
  const int ntiles = last_pos < 0 ? 0 : last_pos / kTileTokens + 1;
  const int nfull = first_pos < 0 ? 0 : (first_pos + 1) / kTileTokens;  // tiles needing no mask

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int li = lane & 15, lk = lane >> 4;
  const int Hq = a.num_q_heads;
  // score scale and output scale of this kv head (per-head dequantisation scales if given).
  // The softmax takes the max of the raw scores and folds the scale into the exponent's
  // fma, which needs a scale >= 0: a negative one is moved onto q (an exact sign flip).
  const float qks_signed =
      a.k_head_scales ? (a.qk_scale * a.k_head_scales[kvh]) * kLog2e : a.qk_scale_log2;
  // (at least the smallest normal float, so that a masked score of -inf times it stays
  // -inf; finite scores times it round to equal weights, as with a zero scale)
  const float qks = fmaxf(fabsf(qks_signed), __FLT_MIN__);
  const uint32_t qflip = qks_signed < 0.0f ? 0x80008000u : 0u;
  const float vsc = a.v_head_scales ? a.v_head_scales[kvh] : a.v_scale;

  // ---- q rows as the B operand: lane (li, lk) holds dims 32c + 8lk .. +7 of row li
  u32x4 qop[RG][NC];
  int qpos[RG];                                            // position of row li's token
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int r = (wave * RG + rg) * 16 + li;
    const int t = t0 + r / G, h = r % G;
    const bool ok = t < nr;
    qpos[rg] = pos0 + (ok ? t : nr - 1);                   // padding rows copy a real one
    // padding rows load the last real row (finite scores; never stored)
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                          ((size_t)(qs0 + (ok ? t : nr - 1)) * Hq + (size_t)kvh * G + h) * D * 2;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qop[rg][c] = *reinterpret_cast<const u32x4*>(qrow + (32 * c + 8 * lk) * 2) ^ qflip;
  }
  // Wait for q here, once: an empty asm that reads and redefines the registers makes the
  // compiler place that wait now, instead of waiting for every load in flight at the
  // first use inside the key loop.
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qop[rg][c]));

  // ---- K/V staging. Wave w stages block 4kt + w of tile kt: lane l moves NLD 16-byte
  // pieces, piece j holding row j * RPL + l / TPC at bytes (l % TPC) * 16 .. + 15 of the
  // kv head's row (TPC lanes per row), through one scalar descriptor per block whose size
  // stops at position L, so later rows read as zero (stale or NaN slots never meet a
  // p = 0) and a missing block costs nothing.
  static_assert(kPrefillWaves == 4, "one wave per block of a 64-token tile");
  constexpr int TPC = ROWB / 16;                 // lanes per token row
  constexpr int RPL = kWave / TPC;               // token rows per load instruction
  constexpr int NLD = kBlockTokens / RPL;        // loads per lane, block and pool
  static_assert(TPC * 16 == ROWB && RPL * TPC == kWave && NLD * RPL == kBlockTokens,
                "whole rows per load");
  const uint32_t tok_stride = (uint32_t)a.num_kv_heads * ROWB;
  const size_t blk_stride = (size_t)kBlockTokens * tok_stride;
  const uint8_t* const kpool = static_cast<const uint8_t*>(a.k_pool) + (size_t)kvh * ROWB;
  const uint8_t* const vpool = static_cast<const uint8_t*>(a.v_pool) + (size_t)kvh * ROWB;
  uint32_t ld_off[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j)
    ld_off[j] = (uint32_t)(j * RPL + lane / TPC) * tok_stride + (uint32_t)(lane % TPC) * 16u;
  // KDMA: lane l of load j writes LDS row j * RPL + l / TPC, slot l % TPC, so it fetches the
  // chunk that the swizzle puts there
  uint32_t ldk_off[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int row = j * RPL + lane / TPC;
    ldk_off[j] = (uint32_t)row * tok_stride + (uint32_t)((lane % TPC) ^ (row & (TPC - 1))) * 16u;
  }
  // the block id of wave w's block in tile kt (table entry 4kt + w, the same for every lane
  // of the wave), loaded one tile ahead with the K/V prefetch of the tile before, so its
  // wait is the one the K/V data already takes; entries at or past nb read as 0 and are
  // never used
  const __amdgpu_buffer_rsrc_t rt =
      make_rsrc(a.block_tables + (size_t)b * a.max_blocks_per_seq, (uint32_t)nb * 4u);
  auto load_id = [&](int kt) -> uint32_t { return buf_load4(rt, (uint32_t)(kt * 4 + wave) * 4u); };
  // K of wave w's block in tile kt into registers, or for 16-bit K straight into LDS
  // buffer kt & 1 (its V descriptor kept for stage_v); returns whether the block lies below L with an id outside the pool (never read; its
  // 16 tokens are masked out of the softmax). The V loads are issued later, after the
  // tile's score MFMAs: the four waves of a workgroup reach the staging together after
  // each barrier, and half of their loads then queue at the CU's address unit at once
  // instead of all of them.
  __amdgpu_buffer_rsrc_t rv_next = make_rsrc(vpool, 0u);
  auto stage = [&](int kt, uint32_t id, u32x4 (&kr)[NLD]) -> bool {
    const int rem = L - (kt * 4 + wave) * kBlockTokens;   // rows of the block below L
    const uint32_t pid = (uint32_t)uni((int)id);
    const bool ok = rem > 0 && pid < (uint32_t)a.num_blocks;
    // (selects, not branches: the scalar unit computes both sides)
    const size_t base = (size_t)(ok ? pid : 0u) * blk_stride;
    const uint32_t rows = (uint32_t)(rem < kBlockTokens ? rem : kBlockTokens);
    const uint32_t bytes = ok ? (rows - 1u) * tok_stride + ROWB : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + base, bytes);
    rv_next = make_rsrc(vpool + base, bytes);
    if constexpr (KDMA) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        buf_load16_lds(rk, &s_k[kt & 1][(kBlockTokens * wave + j * RPL) * LROW], ldk_off[j]);
    } else {
#pragma unroll
      for (int j = 0; j < NLD; ++j) kr[j] = buf_load16(rk, ld_off[j]);
    }
    return rem > 0 && !ok;
  };
  auto stage_v = [&](u32x4 (&vr)[NLD]) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) vr[j] = buf_load16(rv_next, ld_off[j]);
  };
  // per LDS buffer, one byte per wave: its block of the tile staged there is out of pool
  __shared__ uint32_t s_bad[2];
  // V rows go to LDS as fp16 for the P.V matrix cores: fp16 and fp8 (exactly widened) as
  // they are, bf16 converted (exact for every |v| below 2^16, the tiniest values aside,
  // which move by less than 2^-25; a larger one becomes an infinity, and so does its
  // product with any weight, or a NaN with a weight of 0: the accumulators are checked
  // once at the end, see below).
  auto to_lds = [&](int buf, const u32x4 (&kr)[NLD], const u32x4 (&vr)[NLD], bool bad,
                    auto fb_tag) {
    constexpr bool FB = decltype(fb_tag)::value;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int tok = kBlockTokens * wave + j * RPL + lane / TPC;
      const int col = (lane % TPC) * 16 * (KV == PA_FP8_E4M3 ? 2 : 1);
      const int at = tok * LROW + col, atv = tok * VROW + col;
      if constexpr (KV == PA_FP8_E4M3) {
        // 16 E4M3 values -> 16 bf16 (K) and 16 fp16 (V), both exact
        u32x4 kx[2], vx[2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          kx[w / 2][2 * (w % 2)] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[j][w], 1.0f, false));
          kx[w / 2][2 * (w % 2) + 1] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(kr[j][w], 1.0f, true));
          vx[w / 2][2 * (w % 2)] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vr[j][w], 1.0f, false));
          vx[w / 2][2 * (w % 2) + 1] = __builtin_bit_cast(
              uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vr[j][w], 1.0f, true));
        }
        *reinterpret_cast<u32x4*>(&s_k[buf][at]) = kx[0];
        *reinterpret_cast<u32x4*>(&s_k[buf][at + 16]) = kx[1];
        *reinterpret_cast<u32x4*>(&s_v[buf][atv]) = vx[0];
        *reinterpret_cast<u32x4*>(&s_v[buf][atv + 16]) = vx[1];
      } else {
        if constexpr (!KDMA) *reinterpret_cast<u32x4*>(&s_k[buf][at]) = kr[j];
        if constexpr (KV == PA_BF16 && !FB) {
          u32x4 vx;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            vx[w] = pack_f16(__uint_as_float(vr[j][w] << 16),
                             __uint_as_float(vr[j][w] & 0xffff0000u));
          }
          *reinterpret_cast<u32x4*>(&s_v[buf][atv]) = vx;
        } else {
          *reinterpret_cast<u32x4*>(&s_v[buf][atv]) = vr[j];
        }
      }
    }
    if (lane == 0) reinterpret_cast<uint8_t*>(&s_bad[buf])[wave] = bad ? 1 : 0;
  };

  // ---- running state: row li's reference max m (log2 units; the running max, moved only
  // when the max outgrows it by more than kLazyMax); acc[rg][e]: lane (j, g) holds rows
  // 4g + v, dim 16e + j; lsum[rg]: lane (j, g) holds the normaliser of rows 4g + v (P
  // times a column of ones on the matrix cores: the sum of exactly the weights P.V takes)
  float m[RG];
  f32x4 acc[RG][DPL], lsum[RG];

  // one key tile: scores, `after_scores` (once the score MFMAs are issued), online
  // softmax, P.V. MASKED: positions past a row's own, and the
  // blocks flagged in `bad` (byte s nonzero: block s of the tile lies outside the pool), get
  // weight 0. FB: V staged as bf16, p as hi + lo bf16 parts.
  auto compute = [&](int buf, int kt, int bad, auto masked_tag, auto fb_tag,
                     auto&& after_scores) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    constexpr bool FB = decltype(fb_tag)::value;
    constexpr int PT = FB ? PA_BF16 : PA_F16;           // element type of the P.V MFMAs
    const uint8_t* Kt = s_k[buf];
    const uint8_t* Vt = s_v[buf];
    // scores: sc[rg][s][v] = row li of group rg against token 16s + 4lk + v
    f32x4 sc[RG][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 kop[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kop[c] = *reinterpret_cast<const u32x4*>(
            Kt + (16 * s + li) * LROW +
            (KDMA ? ((4 * c + lk) ^ (li & (TPC - 1))) * 16 : (32 * c + 8 * lk) * 2));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NC; ++c) z = mfma32<ST>(kop[c], qop[rg][c], z);
        sc[rg][s] = z;
      }
    }
    after_scores();
    u32x4 aop[RG][2];                      // P as the A operand, two subtiles per MFMA
    u32x4 alo[FB ? RG : 1][2];             // the low parts of P (FB)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      // raw scores; the max commutes with the (non-negative) scale, rounding included
      bool live[4][4];
      float bm = neg_inf();
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          live[s][v] = !MASKED || (kt * kTileTokens + 16 * s + 4 * lk + v <= qpos[rg] &&
                                   !((bad >> (8 * s)) & 1));
          bm = fmaxf(bm, live[s][v] ? sc[rg][s][v] : neg_inf());
        }
      const float mx = xrow_max(fmaxf(bm * qks, m[rg]));   // the row's running max
      const float mn = mx > m[rg] + kLazyMax ? mx : m[rg];  // its reference (-inf at first)
      const float base = mn == neg_inf() ? 0.0f : mn;
      // p = 2^(s * scale - max); masked positions are 0 (also for a zero scale)
      float sv[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[s][v] = fmaf(sc[rg][s][v], qks, -base);
#pragma unroll
      for (int pi = 0; pi < 2; ++pi) {
        uint32_t w[4], wl[4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 4; v += 2) {
            float pa = fast_exp2(sv[2 * pi + h][v]);
            float pb = fast_exp2(sv[2 * pi + h][v + 1]);
            if constexpr (MASKED) {
              pa = live[2 * pi + h][v] ? pa : 0.0f;
              pb = live[2 * pi + h][v + 1] ? pb : 0.0f;
            }
            if constexpr (FB) {
              const uint32_t ua = __float_as_uint(pa), ub = __float_as_uint(pb);
              w[2 * h + v / 2] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // high halves
              wl[2 * h + v / 2] = pack_bf16(pa - __uint_as_float(ua & 0xffff0000u),
                                            pb - __uint_as_float(ub & 0xffff0000u));
            } else {
              w[2 * h + v / 2] = pack_f16(pa, pb);
            }
          }
        aop[rg][pi] = u32x4{w[0], w[1], w[2], w[3]};
        if constexpr (FB) alo[rg][pi] = u32x4{wl[0], wl[1], wl[2], wl[3]};
      }
      const float mold = m[rg];
      m[rg] = mn;
      // rows 4lk + v of the accumulators take the factor of row 4lk + v (held by lane 4lk + v),
      // worked out only when some row's reference moved
      if (__builtin_amdgcn_ballot_w64(mn != mold) != 0) {
        const float al = mn == mold ? 1.0f : fast_exp2(mold - base);
        float alv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) alv[v] = __shfl(al, 4 * lk + v);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[rg][e][v] *= alv[v];
          lsum[rg][v] *= alv[v];
        }
      }
    }
    // P.V: k-slot 8lk + i is token 32pi + 4lk + i (i < 4) or 32pi + 16 + 4lk + i - 4, and
    // MFMA e covers output dims 16e + n (column n). Its B operand, dim 16e + n of those
    // eight tokens, comes from two transposed LDS reads (ds_read_b64_tr_b16): in each
    // 16-lane group lane i receives element i % 4 of the 8-byte rows that lanes i / 4,
    // i / 4 + 4, i / 4 + 8 and i / 4 + 12 point at, so lane R points at token t0 + R / 4,
    // dims 16e + 4 (R % 4) .. + 3, and lane n gets dim 16e + n of tokens t0 .. t0 + 3.
    // A B operand of ones (1.0 in PT) adds each row's weights to lsum.
    const uint32_t one2 = PT == PA_F16 ? 0x3c003c00u : 0x3f803f80u;
    const u32x4 ones = {one2, one2, one2, one2};
    const int tq = li >> 2, dq = 4 * (li & 3);
#pragma unroll
    for (int pi = 0; pi < 2; ++pi) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        lsum[rg] = mfma32<PT>(aop[rg][pi], ones, lsum[rg]);
        if constexpr (FB) lsum[rg] = mfma32<PT>(alo[rg][pi], ones, lsum[rg]);
      }
      const uint8_t* vrow = Vt + (32 * pi + 4 * lk + tq) * VROW + dq * 2;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vrow + 32 * e));
        const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vrow + 16 * VROW + 32 * e));
        const u32x2 w0 = __builtin_bit_cast(u32x2, b0), w1 = __builtin_bit_cast(u32x2, b1);
        const u32x4 bop = {w0[0], w0[1], w1[0], w1[1]};
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          acc[rg][e] = mfma32<PT>(aop[rg][pi], bop, acc[rg][e]);
          if constexpr (FB) acc[rg][e] = mfma32<PT>(alo[rg][pi], bop, acc[rg][e]);
        }
      }
    }
  };

  // ---- the key loop: stage tile kt + 1 (ids one tile further ahead) while computing kt.
  // Tiles wholly at or before the first query position need no mask, unless a block of
  // theirs lies outside the pool; from the first tile that needs one on, all take the
  // masked body. Two loops, so that each body is compiled (and its registers allocated)
  // on its own.
  auto run = [&](auto fb_tag) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      m[rg] = neg_inf();
      lsum[rg] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[rg][e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    uint32_t id = 0;
    u32x4 kr[NLD], vr[NLD];
    bool bad = false;
    if (ntiles > 0) {
      id = load_id(0);
      bad = stage(0, id, kr);
      stage_v(vr);
      id = load_id(1);
      to_lds(0, kr, vr, bad, fb_tag);
    }
    if constexpr (KDMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // K landed in LDS
    __syncthreads();
    auto step = [&](int kt, auto masked_tag) {
      const bool more = kt + 1 < ntiles;
      // (KDMA: the next tile's K is requested after this tile's score MFMAs, so that it
      // lands in LDS while the softmax and P.V run rather than under the score phase's
      // operand reads)
      if (more && !KDMA) {
        bad = stage(kt + 1, id, kr);
        id = load_id(kt + 2);
      }
      compute(kt & 1, kt, (int)s_bad[kt & 1], masked_tag, fb_tag, [&]() {
        if (more) {
          if constexpr (KDMA) {
            bad = stage(kt + 1, id, kr);
            id = load_id(kt + 2);
          }
          stage_v(vr);
        }
      });
      if (more) to_lds((kt + 1) & 1, kr, vr, bad, fb_tag);
      if constexpr (KDMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // K landed in LDS
      __syncthreads();
    };
    const int nfree = nfull < ntiles ? nfull : ntiles;
    int kt = 0;
    for (; kt < nfree && s_bad[kt & 1] == 0; ++kt) step(kt, std::false_type{});
    for (; kt < ntiles; ++kt) step(kt, std::true_type{});
  };
  run(std::false_type{});
  // bf16 V: a value beyond fp16's range (2^16 or more, an infinity or a NaN) has left a
  // non-finite accumulator in some row of the workgroup (its fp16 infinity times a weight,
  // or times a zero weight of a masked position: NaN), while a finite V gives finite sums
  // (weights at most 2^kLazyMax, |v| below 2^16). Such a workgroup runs its key loop again
  // with V staged as bf16 and each weight split into two bf16 parts (FB), and stores only
  // that result.
  if constexpr (KV == PA_BF16) {
    float amax = 0.0f;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int e = 0; e < DPL; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          amax = __builtin_elementwise_maximum(amax, __builtin_fabsf(acc[rg][e][v]));  // NaN-propagating
    if (__syncthreads_or(!(amax <= __FLT_MAX__))) run(std::true_type{});
  }

  // ---- normalise and store: lane (j, lk) writes rows 4lk + v, dims 16e + j
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float lr = lsum[rg][v];
      const int r = (wave * RG + rg) * 16 + 4 * lk + v;
      const int t = t0 + r / G, h = r % G;
      if (t >= nr) continue;
      const float inv = lr > 0.0f ? vsc / lr : 0.0f;
      const size_t o = ((size_t)(qs0 + t) * Hq + (size_t)kvh * G + h) * D + li;
#pragma unroll
      for (int e = 0; e < DPL; ++e) store_out<OT>(a.out, o + 16 * e, acc[rg][e][v] * inv);
    }
  }
}

template <int KV, int OT, int D, int G>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  prefill_kernel<KV, OT, D, G, kPrefillRowGroups><<<dim3(a.num_workgroups), dim3(kPrefillThreads),
                                                   0, stream>>>(a);
  return hipGetLastError();
}

template <int KV, int OT, int D>
hipError_t prefill_group(int group, const PrefillArgs& a, hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_t<KV, OT, D, 1>(a, stream);
    case 2: return launch_prefill_t<KV, OT, D, 2>(a, stream);
    case 4: return launch_prefill_t<KV, OT, D, 4>(a, stream);
    case 8: return launch_prefill_t<KV, OT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, int OT>
hipError_t prefill_dim(int head_dim, int group, const PrefillArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return prefill_group<KV, OT, 64>(group, a, stream);
    case 128: return prefill_group<KV, OT, 128>(group, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                          const PrefillArgs& a, hipStream_t stream) {
  if (q_dtype == PA_F16 && kv_dtype == PA_F16) {
    if (out_dtype == PA_F16) return prefill_dim<PA_F16, PA_F16>(head_dim, group, a, stream);
    if (out_dtype == PA_F32) return prefill_dim<PA_F16, PA_F32>(head_dim, group, a, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_BF16) {
    if (out_dtype == PA_BF16) return prefill_dim<PA_BF16, PA_BF16>(head_dim, group, a, stream);
    if (out_dtype == PA_F32) return prefill_dim<PA_BF16, PA_F32>(head_dim, group, a, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3) {
    if (out_dtype == PA_BF16)
      return prefill_dim<PA_FP8_E4M3, PA_BF16>(head_dim, group, a, stream);
    if (out_dtype == PA_F32) return prefill_dim<PA_FP8_E4M3, PA_F32>(head_dim, group, a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
