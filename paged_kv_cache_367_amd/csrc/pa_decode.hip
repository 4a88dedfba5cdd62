// pa_decode.hip - decode attention over a block-paged KV cache, gfx950 (CDNA4).
//
// What is computed (vLLM-PagedAttention与连续批处理技术拆解, sections 3.1-3.3): every
// sequence's single query attends over its first L tokens, whose K/V rows live in
// 16-token blocks found through the sequence's block table. Softmax is computed block
// by block: each block contributes its local max and normaliser, and running results
// are rescaled whenever the max moves (FlashAttention-style), which equals the global
// softmax exactly in real arithmetic.
//
// How it maps onto CDNA4
//   * Work item = (kv head g, sequence b, partition of P blocks); one workgroup of 4
//     waves per item. Wave w takes the partition's blocks w, w+4, w+8, ...; the G query
//     heads sharing kv head g are all served by the same K/V bytes, read once.
//   * QK^T runs on the matrix cores (v_mfma_f32_16x16x32_{bf16,f16}, fp8 converted to
//     bf16 first, v_mfma_f32_16x16x4f32 for fp32). Operand B is the K block exactly as
//     it sits in HBM: lane (t, q) = (lane % 16, lane / 16) loads 16-byte chunk 4s+q of
//     token t's row, so each load instruction covers 64 contiguous bytes of 16 rows and
//     no shuffle or LDS pass is needed. Operand A repeats the G query rows over the 16
//     MFMA rows (row i holds head i % G), so after the MFMA every lane holds the scores
//     of its token for G distinct heads.
//   * Block max: 16-lane DPP row reduction. Probabilities p[t][h] go to LDS once per
//     block and are read back broadcast by the V stage.
//   * PV on the vector ALU in fp32: lane (r, c) owns 16-byte chunk c of V rows r,
//     r + RPI, ... and accumulates acc[h][e] for all G heads, so every V byte is
//     converted once and used G times. At the end, lanes owning the same chunk are
//     summed (xor shuffles), then the 4 waves are merged through LDS.
//   * One partition covers the whole sequence: the final output is written directly.
//     Otherwise (m, l, acc) go to the workspace and merge_kernel combines them.
//   * The partial last block is masked by selection (scores -> -inf, V -> 0), so stale
//     or NaN slots past L never reach the result.
//   * Reduction order depends on logical positions only, never on physical block ids,
//     so moving blocks in the pool leaves the output bitwise unchanged.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/paged_attention.h"
#include "pa_launch.h"

namespace pa {
namespace {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: after the four
// steps every lane of a 16-lane row holds the row's reduction.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

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
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
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

// One 16-byte K chunk against the matching q piece(s): acc += A(q) * B(k).
template <int KV>
__device__ __forceinline__ f32x4 qk_chunk(f32x4 acc, u32x4 k, const u32x4* qc) {
  if constexpr (KV == PA_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qc[0]),
                                                  __builtin_bit_cast(bf16x8, k), acc, 0, 0, 0);
  } else if constexpr (KV == PA_F16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, qc[0]),
                                                 __builtin_bit_cast(f16x8, k), acc, 0, 0, 0);
  } else if constexpr (KV == PA_FP8_E4M3) {
    // 16 E4M3 values -> two groups of 8 bf16 (exact: every E4M3 value is a bf16 value)
    bf16x2 e[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      e[2 * w] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.0f, false);
      e[2 * w + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[w], 1.0f, true);
    }
    bf16x8 k0 = {e[0][0], e[0][1], e[1][0], e[1][1], e[2][0], e[2][1], e[3][0], e[3][1]};
    bf16x8 k1 = {e[4][0], e[4][1], e[5][0], e[5][1], e[6][0], e[6][1], e[7][0], e[7][1]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qc[0]), k0, acc,
                                                  0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qc[1]), k1, acc,
                                                  0, 0, 0);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(qc[0][e]), __uint_as_float(k[e]),
                                                 acc, 0, 0, 0);
  }
  return acc;
}

// One 16-byte V chunk -> fp32 values.
template <int KV>
__device__ __forceinline__ void v_chunk(u32x4 w, float* v) {
  if constexpr (KV == PA_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else if constexpr (KV == PA_F16) {
    // Cast the whole 16-byte vector: hipcc 7.2 miscompiles a bit_cast of one u32 element
    // to a 2 x half vector inside an unrolled loop (it reuses element 0 for every i).
    const f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  } else if constexpr (KV == PA_FP8_E4M3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
      f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
      v[4 * i] = lo[0];
      v[4 * i + 1] = lo[1];
      v[4 * i + 2] = hi[0];
      v[4 * i + 3] = hi[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(w[i]);
  }
}

__device__ __forceinline__ int clamp_len(int L, int max_blocks_per_seq, int max_context_len) {
  L = L < 0 ? 0 : L;
  int cap = max_blocks_per_seq * kBlockTokens;
  cap = cap < max_context_len ? cap : max_context_len;
  return L < cap ? L : cap;
}

template <int KV, int QT, int OT, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_kernel(DecodeArgs a) {
  constexpr int KB = Enc<KV>::bytes;
  constexpr int QB = Enc<QT>::bytes;
  constexpr int ROWB = D * KB;            // bytes of one token's K (or V) row, one kv head
  constexpr int NL = ROWB / 64;           // 16-byte loads per lane per block, K and V each
  constexpr int EPC = 16 / KB;            // elements per 16-byte chunk
  constexpr int LPR = ROWB / 16;          // V stage: lanes per token row
  constexpr int RPI = kWave / LPR;        // V stage: token rows per load instruction
  constexpr int QROWS = G > 4 ? G / 4 : 1;  // MFMA row groups holding distinct heads
  constexpr int HPL = G < 4 ? G : 4;        // distinct heads per lane after the MFMA
  constexpr int QCH = EPC * QB / 16;        // 16-byte q pieces matching one K chunk
  static_assert(NL >= 1 && NL * RPI == kBlockTokens, "block layout");
  static_assert(QCH >= 1, "q layout");

  constexpr int PBUF = kBlockTokens * G + 8;    // p[16][G] + alpha[8], one block, one wave
  constexpr int LOOP_FLOATS = NW * 2 * PBUF;
  constexpr int COMB_FLOATS = NW * G * (D + 2);
  __shared__ float smem[LOOP_FLOATS > COMB_FLOATS ? LOOP_FLOATS : COMB_FLOATS];

  // Grid (kv head, sequence, partition): workgroups are handed to the 8 XCDs round-robin
  // in linear order, so the kv head varies fastest (for 8 kv heads each XCD serves one
  // head and keeps its slices of shared blocks in its own L2) and the partition slowest
  // (every sequence has partition 0; the empty tail partitions are dispatched last).
  const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // the wave index is uniform within a wave; say so, so that everything derived from it
  // (block ranges, buffer descriptors) stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;

  const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.max_context_len);
  const int nb = (L + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (nb + a.part_blocks - 1) / a.part_blocks;
  if (L == 0) {  // nothing to attend: zero output
    if (part == 0)
      for (int idx = tid; idx < G * D; idx += NW * kWave)
        store_out<OT>(a.out, ((size_t)b * Hq + g * G) * D + idx, 0.0f);
    return;
  }
  if (part >= nparts) return;
  const int jbeg = part * a.part_blocks;
  const int jend = min(nb, jbeg + a.part_blocks);

  // ---- query operand: MFMA row i = lane % 16 carries head i % G; chunk c = 4s + lane/16
  u32x4 qreg[NL][QCH];
  {
    const uint8_t* qrow = static_cast<const uint8_t*>(a.q) +
                          ((size_t)b * Hq + (size_t)g * G + (lane & 15) % G) * D * QB;
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int c = 4 * s + (lane >> 4);
#pragma unroll
      for (int u = 0; u < QCH; ++u)
        qreg[s][u] = *reinterpret_cast<const u32x4*>(qrow + c * EPC * QB + u * 16);
    }
  }

  // ---- this wave's physical block ids, one per lane, read back with readlane
  const int nwb = jend - jbeg - wave > 0 ? (jend - jbeg - wave + NW - 1) / NW : 0;
  int my_id = 0;
  if (lane < nwb)
    my_id = a.block_tables[(size_t)b * a.max_blocks_per_seq + jbeg + wave + NW * lane];

  const uint32_t tok_stride = (uint32_t)Hkv * ROWB;       // bytes between tokens of a block
  const uint32_t blk_stride = kBlockTokens * tok_stride;  // bytes between physical blocks
  const uint8_t* const kpool = static_cast<const uint8_t*>(a.k_pool);
  const uint8_t* const vpool = static_cast<const uint8_t*>(a.v_pool);
  // per-lane byte offsets inside a block (constant over the loop)
  const uint32_t koff = (uint32_t)g * ROWB + (lane & 15) * tok_stride + (lane >> 4) * 16;
  const uint32_t voff = (uint32_t)g * ROWB + (lane / LPR) * tok_stride + (lane % LPR) * 16;

  float m[HPL], lsum[HPL];
#pragma unroll
  for (int r = 0; r < HPL; ++r) {
    m[r] = neg_inf();
    lsum[r] = 0.0f;
  }
  float acc[G][EPC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;

  float* const pw = smem + wave * 2 * PBUF;  // this wave's two p/alpha buffers

  // Issue the loads of the wave's k-th block. Always issues the same instructions so the
  // compiler's wait counts stay static; k >= nwb (or a bad block id) loads from an
  // empty descriptor and yields zeros without memory traffic.
  auto issue = [&](int k, u32x4(&kb)[NL], u32x4(&vb)[NL], bool& valid) {
    const bool real = k < nwb;
    const int pid = __builtin_amdgcn_readlane(my_id, real ? k : 0);
    valid = real && (unsigned)pid < (unsigned)a.num_blocks;
    const size_t base = valid ? (size_t)pid * blk_stride : 0;
    const uint32_t bytes = valid ? blk_stride : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + base, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vpool + base, bytes);
#pragma unroll
    for (int s = 0; s < NL; ++s) kb[s] = buf_load16(rk, koff + s * 64);
#pragma unroll
    for (int i = 0; i < NL; ++i) vb[i] = buf_load16(rv, voff + i * RPI * tok_stride);
  };
  auto compute = [&](int j, bool valid, const u32x4(&kb)[NL], const u32x4(&vb)[NL],
                     float* P) {
    // scores of token t = lane % 16 for the heads of MFMA rows 4*(lane/16) + r
    f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NL; ++s) sc = qk_chunk<KV>(sc, kb[s], qreg[s]);
    const bool ragged = !valid || (j + 1) * kBlockTokens > L;
    const bool tok_ok = valid && (j * kBlockTokens + (lane & 15) < L);
    float al[HPL], p[HPL];
#pragma unroll
    for (int r = 0; r < HPL; ++r) {
      float s = sc[r] * a.qk_scale_log2;
      if (ragged) s = tok_ok ? s : neg_inf();
      const float mn = fmaxf(m[r], row16_max(s));
      al[r] = mn == neg_inf() ? 1.0f : fast_exp2(m[r] - mn);
      p[r] = fast_exp2(s - mn);
      if (ragged) p[r] = tok_ok ? p[r] : 0.0f;
      lsum[r] = lsum[r] * al[r] + p[r];
      m[r] = mn;
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
        for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h];
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = lane / LPR + RPI * i;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = P[row * G + h];
      float v[EPC];
      v_chunk<KV>(vb[i], v);
      if (ragged) {
        const bool ok = valid && (j * kBlockTokens + row < L);
#pragma unroll
        for (int e = 0; e < EPC; ++e) v[e] = ok ? v[e] : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
    }
  };

  // ---- main loop over this wave's blocks: two register buffers, the next block's
  // loads always in flight while the current block is computed
  if (nwb > 0) {
    u32x4 k0[NL], v0[NL], k1[NL], v1[NL];
    bool val0, val1;
    issue(0, k0, v0, val0);
    issue(1, k1, v1, val1);
    for (int k = 0; k < nwb; k += 2) {
      const int j0 = jbeg + wave + NW * k;
      compute(j0, val0, k0, v0, pw);
      issue(k + 2, k0, v0, val0);
      if (k + 1 < nwb) compute(j0 + NW, val1, k1, v1, pw + PBUF);
      issue(k + 3, k1, v1, val1);
    }
  }

  // ---- combine: lanes of a row (lsum), lanes sharing a V chunk (acc), then waves
#pragma unroll
  for (int r = 0; r < HPL; ++r) lsum[r] = row16_sum(lsum[r]);
#pragma unroll
  for (int st = LPR; st < kWave; st <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], st);

  __syncthreads();  // every wave is done with its loop buffers
  float* Wm = smem;
  float* Wl = smem + NW * G;
  float* Wa = smem + 2 * NW * G;
  if ((lane & 15) == 0 && (lane >> 4) < QROWS) {
    const int hb = G > 4 ? 4 * (lane >> 4) : 0;
#pragma unroll
    for (int r = 0; r < HPL; ++r) {
      Wm[wave * G + hb + r] = m[r];
      Wl[wave * G + hb + r] = lsum[r];
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) Wa[(wave * G + h) * D + EPC * lane + e] = acc[h][e];
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += NW * kWave) {
    const int h = idx / D, dd = idx % D;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, Wm[w * G + h]);
    float Ls = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = Wm[w * G + h];
      const float f = mw == neg_inf() ? 0.0f : fast_exp2(mw - M);
      Ls = fmaf(Wl[w * G + h], f, Ls);
      A = fmaf(Wa[(w * G + h) * D + dd], f, A);
    }
    const size_t hq = (size_t)b * Hq + (size_t)g * G + h;
    if (nparts == 1) {
      store_out<OT>(a.out, hq * D + dd, Ls > 0.0f ? a.v_scale * (A / Ls) : 0.0f);
    } else {
      const size_t slot = hq * a.max_parts + part;
      a.ws_acc[slot * D + dd] = A;
      if (dd == 0) {
        a.ws_ml[slot * 2] = M;
        a.ws_ml[slot * 2 + 1] = Ls;
      }
    }
  }
}

// Cross-partition merge with the same rescaling: M = max_p m_p,
// out = v_scale * sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
template <int OT, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int hq = blockIdx.x * 4 + wave, b = blockIdx.y;
  if (hq >= a.num_q_heads) return;
  const int L = clamp_len(a.context_lens[b], a.max_blocks_per_seq, a.max_context_len);
  const int nb = (L + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (nb + a.part_blocks - 1) / a.part_blocks;
  if (nparts <= 1) return;
  const size_t base = ((size_t)b * a.num_q_heads + hq) * a.max_parts;
  const float* ml = a.ws_ml + base * 2;
  const float* acc = a.ws_acc + base * D;
  float M = neg_inf();
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  constexpr int PER = D / kWave;
  float A[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) A[k] = 0.0f;
  float Ls = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float mp = ml[2 * p];
    const float f = mp == neg_inf() ? 0.0f : fast_exp2(mp - M);
    Ls = fmaf(ml[2 * p + 1], f, Ls);
#pragma unroll
    for (int k = 0; k < PER; ++k) A[k] = fmaf(acc[(size_t)p * D + lane + kWave * k], f, A[k]);
  }
  const size_t o = ((size_t)b * a.num_q_heads + hq) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    store_out<OT>(a.out, o + lane + kWave * k, Ls > 0.0f ? a.v_scale * (A[k] / Ls) : 0.0f);
}

template <int KV, int QT, int OT, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& args, int batch, hipStream_t stream) {
  dim3 grid(args.num_kv_heads, batch, args.max_parts);
  decode_kernel<KV, QT, OT, D, G, kDecodeWaves><<<grid, kDecodeWaves * kWave, 0, stream>>>(args);
  return hipGetLastError();
}

template <int KV, int QT, int OT, int D>
hipError_t dispatch_group(int group, const DecodeArgs& args, int batch, hipStream_t stream) {
  switch (group) {
    case 1: return launch_decode_t<KV, QT, OT, D, 1>(args, batch, stream);
    case 2: return launch_decode_t<KV, QT, OT, D, 2>(args, batch, stream);
    case 4: return launch_decode_t<KV, QT, OT, D, 4>(args, batch, stream);
    case 8: return launch_decode_t<KV, QT, OT, D, 8>(args, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int KV, int QT, int OT>
hipError_t dispatch_dim(int head_dim, int group, const DecodeArgs& args, int batch,
                        hipStream_t stream) {
  switch (head_dim) {
    case 64: return dispatch_group<KV, QT, OT, 64>(group, args, batch, stream);
    case 128: return dispatch_group<KV, QT, OT, 128>(group, args, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(int q_dtype, int kv_dtype, int out_dtype, int head_dim, int group,
                         const DecodeArgs& args, int batch, hipStream_t stream) {
  if (q_dtype == PA_F32 && kv_dtype == PA_F32 && out_dtype == PA_F32)
    return dispatch_dim<PA_F32, PA_F32, PA_F32>(head_dim, group, args, batch, stream);
  if (q_dtype == PA_F16 && kv_dtype == PA_F16) {
    if (out_dtype == PA_F16)
      return dispatch_dim<PA_F16, PA_F16, PA_F16>(head_dim, group, args, batch, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_F16, PA_F16, PA_F32>(head_dim, group, args, batch, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_BF16) {
    if (out_dtype == PA_BF16)
      return dispatch_dim<PA_BF16, PA_BF16, PA_BF16>(head_dim, group, args, batch, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_BF16, PA_BF16, PA_F32>(head_dim, group, args, batch, stream);
  }
  if (q_dtype == PA_BF16 && kv_dtype == PA_FP8_E4M3) {
    if (out_dtype == PA_BF16)
      return dispatch_dim<PA_FP8_E4M3, PA_BF16, PA_BF16>(head_dim, group, args, batch, stream);
    if (out_dtype == PA_F32)
      return dispatch_dim<PA_FP8_E4M3, PA_BF16, PA_F32>(head_dim, group, args, batch, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int out_dtype, int head_dim, const MergeArgs& args, int batch,
                        hipStream_t stream) {
  dim3 grid((args.num_q_heads + 3) / 4, batch);
  dim3 block(256);
#define PA_MERGE(OT, D) merge_kernel<OT, D><<<grid, block, 0, stream>>>(args)
  if (head_dim == 64) {
    if (out_dtype == PA_F32) PA_MERGE(PA_F32, 64);
    else if (out_dtype == PA_F16) PA_MERGE(PA_F16, 64);
    else PA_MERGE(PA_BF16, 64);
  } else {
    if (out_dtype == PA_F32) PA_MERGE(PA_F32, 128);
    else if (out_dtype == PA_F16) PA_MERGE(PA_F16, 128);
    else PA_MERGE(PA_BF16, 128);
  }
#undef PA_MERGE
  return hipGetLastError();
}

}  // namespace pa
