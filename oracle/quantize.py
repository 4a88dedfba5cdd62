"""Quantisation of new K/V rows to OCP fp8 E4M3FN on the slot write (oracle; test
infrastructure).

The pages say that setting the KV cache dtype to fp8 (E4M3) halves the KV cache memory
(vLLM-PagedAttention与连续批处理技术拆解, section 五, the flag table and the KV cache
quantisation note); they do not fix how values are scaled or rounded. Reading taken
here, shared with the decode's per-tensor dequantisation scale s (stored value =
code value * s):

  inv  = fp32(1 / s)                       (one binary32 division)
  y    = fp32(fp32(x) * inv)               (one binary32 multiply, round to nearest even)
  code = E4M3(y)                           (e4m3_encode below)

so that both sides make the rounding decision from the same binary32 number.

e4m3_encode, from the format definition (1 sign bit, 4 exponent bits with bias 7, 3
mantissa bits, exponent 0 subnormal, S.1111.111 NaN, largest finite 448):
  - NaN -> 0x7F;
  - |y| >= 448, infinities included -> +-448 (saturation);
  - otherwise the nearest of the 127 finite non-negative values, ties to the code with
    an even mantissa, with y's sign bit (so -0.0 and negative values that round to zero
    give 0x80).
Values are compared as float64 against the decode table, which holds every E4M3 value
exactly, so the nearest-value search itself makes no rounding error.
"""
from __future__ import annotations

import numpy as np

from .storage import decode_storage, e4m3_table

E4M3_MAX = 448.0


def quant_inputs(new: np.ndarray, kind: str, scale) -> np.ndarray:
    """The binary32 values y = fp32(fp32(x) * fp32(1 / scale)) that get encoded; new is
    [T, Hkv, d] and scale one number or one per kv head (head g divided by its own)."""
    x = decode_storage(new, kind).astype(np.float32)        # exact: every source is binary32-representable
    s = np.asarray(scale, dtype=np.float32).reshape(-1)
    if s.size == 1:
        inv = np.float32(1.0) / s[0]                        # one binary32 division
    elif x.ndim >= 2 and s.size == x.shape[-2]:
        inv = (np.float32(1.0) / s).reshape(-1, 1)          # one per kv head
    else:
        raise ValueError("one scale, or one per kv head")
    with np.errstate(over="ignore", invalid="ignore"):
        return x * inv


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float values -> E4M3FN codes (uint8), by nearest-value search over the code table."""
    y = np.asarray(y, dtype=np.float64)
    vals = e4m3_table()[:127]                    # codes 0x00..0x7E: 0 .. 448, increasing
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i, v in enumerate(flat):
        if np.isnan(v):
            out[i] = 0x7F
            continue
        sign = 0x80 if np.signbit(v) else 0x00
        a = abs(v)
        if a >= E4M3_MAX:
            out[i] = sign | 0x7E
            continue
        hi = int(np.searchsorted(vals, a, side="left"))   # first value >= a
        if vals[hi] == a:
            code = hi
        else:
            lo = hi - 1
            dlo, dhi = a - vals[lo], vals[hi] - a
            if dlo < dhi:
                code = lo
            elif dhi < dlo:
                code = hi
            else:
                code = lo if lo % 2 == 0 else hi          # the even mantissa
        out[i] = sign | code
    return out.reshape(y.shape)


def cache_write_fp8_ref(pool: np.ndarray, new: np.ndarray, kind: str, scale,
                        slot_mapping: np.ndarray) -> np.ndarray:
    """fp8 pool [N, bs, Hkv, d] (uint8), new rows [T, Hkv, d] in storage encoding `kind`
    (f32, f16 or bf16 bits), dequantisation scale (per tensor, or per kv head), slots [T]
    (-1 = skip) ->
    updated copy of the pool with row s written as the E4M3 codes of the new row."""
    N, bs = pool.shape[:2]
    out = np.array(pool, dtype=np.uint8, copy=True)
    codes = e4m3_encode(quant_inputs(new, kind, scale))
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        if s >= N * bs:
            raise ValueError("slot outside the pool")
        out[s // bs, s % bs] = codes[t]
    return out
