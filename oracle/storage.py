"""Decode stored KV / query encodings to float64 (oracle; test infrastructure).

fp32 and fp16 are IEEE binary32 / binary16 and widen exactly. bf16 is the upper half
of a binary32 word. fp8 is OCP E4M3FN, the format the "--kv-cache-dtype fp8" flag
selects (vLLM-PagedAttention与连续批处理技术拆解, section 五, flag table and the FP8 note):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, exponent 0 subnormal,
S.1111.111 NaN, no infinities, largest finite value 448.
"""
from __future__ import annotations

import numpy as np

_E4M3_CACHE = None


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: place them in the high half of a binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # signalling-NaN patterns widen to NaN
        return u.view(np.float32).astype(np.float64)


def e4m3_table() -> np.ndarray:
    """All 256 E4M3FN code points as float64, built from the format definition."""
    global _E4M3_CACHE
    if _E4M3_CACHE is None:
        t = np.empty(256, dtype=np.float64)
        for code in range(256):
            sign = -1.0 if (code >> 7) & 1 else 1.0
            exp = (code >> 3) & 0xF
            man = code & 0x7
            if exp == 0xF and man == 0x7:
                t[code] = np.nan
            elif exp == 0:
                t[code] = sign * (man / 8.0) * 2.0 ** (1 - 7)
            else:
                t[code] = sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)
        _E4M3_CACHE = t
    return _E4M3_CACHE


def decode_storage(arr: np.ndarray, kind: str) -> np.ndarray:
    """Storage array of encoding `kind` -> float64 array of the same shape."""
    if kind == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if kind == "f16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    if kind == "bf16":
        return bf16_bits_to_f64(arr)
    if kind == "fp8_e4m3":
        return e4m3_table()[np.asarray(arr, dtype=np.uint8)]
    raise ValueError(f"unknown storage kind {kind!r}")
