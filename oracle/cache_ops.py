"""Slot write and copy-on-write block copy, reference versions (oracle; test infrastructure).

cache_write_ref: a generated token occupies one slot (vLLM-PagedAttention与连续批处理技术
拆解, section 3.1); slot s is block s // block_size, row s % block_size of the pool.
block_copy_ref: a shared block is read-only and a sequence that must write into it
copies it first (same page, section 3.4; serving-engine article, section 2, shared
blocks). Both are pure bit copies; they work on unsigned-integer views so that NaN
payloads and signed zeros are preserved exactly.
"""
from __future__ import annotations

import numpy as np


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


def cache_write_ref(pool: np.ndarray, new: np.ndarray, slot_mapping: np.ndarray) -> np.ndarray:
    """pool [N, bs, Hkv, d], new [T, Hkv, d], slots [T] (-1 = skip) -> updated copy."""
    N, bs = pool.shape[:2]
    out = pool.copy()
    ob, nb = _bits(out), _bits(np.ascontiguousarray(new))
    for t, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        if s >= N * bs:
            raise ValueError("slot outside the pool")
        ob[s // bs, s % bs] = nb[t]
    return out


def block_copy_ref(pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """pool [N, ...], pairs [P, 2] of (src, dst) -> copy with pool[dst] = old pool[src]."""
    out = pool.copy()
    src_state, ob = _bits(pool), _bits(out)
    for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        ob[d] = src_state[s]
    return out


def block_swap_ref(dst_pool: np.ndarray, src_pool: np.ndarray, pairs: np.ndarray) -> np.ndarray:
    """Whole blocks from one pool to another (swap-out to host memory, swap-in back):
    returns a copy of dst_pool with dst_pool[d] = src_pool[s] for every (s, d) in pairs
    (vLLM-PagedAttention与连续批处理技术拆解, section 4.3, preemption by swapping). Pairs with
    an id outside either pool are skipped."""
    if dst_pool.shape[1:] != src_pool.shape[1:]:
        raise ValueError("pools differ in block shape")
    out = np.array(dst_pool, copy=True)
    for s, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= s < src_pool.shape[0] and 0 <= d < dst_pool.shape[0]:
            out[d] = src_pool[s]
    return out
