"""ctypes binding of the host-side KV block manager in libpa.so (include/pa_block_manager.h).

Argument marshalling only: every decision (allocation, reference counts, copy-on-write,
prefix-cache keys, eviction) is made by the native manager.
"""
from __future__ import annotations

import ctypes

import numpy as np

from .binding import PaError, load_library

PA_ERR_NO_BLOCKS = -8
PA_ERR_UNKNOWN_SEQ = -9

_READY = False


def _lib():
    global _READY
    lib = load_library()
    if not _READY:
        P, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        pi32 = ctypes.POINTER(ctypes.c_int32)
        pi64 = ctypes.POINTER(ctypes.c_int64)
        lib.pa_bm_create.restype = P
        lib.pa_bm_create.argtypes = [I32, I32, I32]
        lib.pa_bm_destroy.restype = None
        lib.pa_bm_destroy.argtypes = [P]
        lib.pa_bm_add.restype = I32
        lib.pa_bm_add.argtypes = [P, I64, pi32, I32, U64, pi32]
        lib.pa_bm_append.restype = I32
        lib.pa_bm_append.argtypes = [P, I64, I32, pi64, pi64, pi64]
        lib.pa_bm_append_batch.restype = I32
        lib.pa_bm_append_batch.argtypes = [P, pi64, pi32, I32, pi64, pi64, pi32, pi32]
        lib.pa_bm_fork.restype = I32
        lib.pa_bm_fork.argtypes = [P, I64, I64]
        lib.pa_bm_free.restype = I32
        lib.pa_bm_free.argtypes = [P, I64]
        lib.pa_bm_slots.restype = I32
        lib.pa_bm_slots.argtypes = [P, I64, I32, I32, pi64]
        lib.pa_bm_block_table.restype = I32
        lib.pa_bm_block_table.argtypes = [P, I64, pi32, I32]
        lib.pa_bm_tables.restype = I32
        lib.pa_bm_tables.argtypes = [P, pi64, I32, pi32, I32, pi32]
        lib.pa_bm_seq_len.restype = I32
        lib.pa_bm_seq_len.argtypes = [P, I64]
        lib.pa_bm_refcount.restype = I32
        lib.pa_bm_refcount.argtypes = [P, I32]
        lib.pa_bm_block_key.restype = I32
        lib.pa_bm_block_key.argtypes = [P, I64, I32, ctypes.POINTER(U64)]
        lib.pa_bm_stats.restype = I32
        lib.pa_bm_stats.argtypes = [P, pi32, pi32, pi32]
        lib.pa_bm_evictable.restype = I32
        lib.pa_bm_evictable.argtypes = [P, pi32, I32]
        lib.pa_bm_set_host_blocks.restype = I32
        lib.pa_bm_set_host_blocks.argtypes = [P, I32]
        lib.pa_bm_swap_out.restype = I32
        lib.pa_bm_swap_out.argtypes = [P, I64, pi64, I32]
        lib.pa_bm_swap_in.restype = I32
        lib.pa_bm_swap_in.argtypes = [P, I64, pi64, I32]
        lib.pa_bm_host_free.restype = I32
        lib.pa_bm_host_free.argtypes = [P]
        _READY = True
    return lib


def _check(st, where):
    if st < 0:
        raise PaError(st, where)
    return st


def _i32p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _i64p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


class BlockManager:
    """Owns one native manager handle (destroyed with the object)."""

    def __init__(self, num_blocks: int, block_size: int = 16, prefix_cache: bool = True):
        self._lib = _lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size), int(prefix_cache))
        if not self._h:
            raise ValueError("pa_bm_create rejected its arguments")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def add(self, seq_id: int, tokens, salt: int = 0) -> int:
        """Add a sequence with its prompt; returns the number of cached prompt tokens."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32(0)
        _check(self._lib.pa_bm_add(self._h, int(seq_id), _i32p(t), t.size,
                                   int(salt) & ((1 << 64) - 1), ctypes.byref(cached)),
               "pa_bm_add")
        return cached.value

    def append(self, seq_id: int, token: int):
        """Append one token; returns (slot, cow_src, cow_dst) with (-1, -1) when no copy."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self._lib.pa_bm_append(self._h, int(seq_id), int(token), ctypes.byref(slot),
                                      ctypes.byref(src), ctypes.byref(dst)), "pa_bm_append")
        return slot.value, src.value, dst.value

    def append_batch(self, seq_ids, tokens):
        """One step's appends in one call: returns (slots int64 [n], cow pairs int64 [k, 2]).
        On a failure raises PaError with .done = the number of appends applied."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        if ids.shape != tok.shape:
            raise ValueError("one token per sequence id")
        slots = np.empty(ids.size, dtype=np.int64)
        pairs = np.empty((max(ids.size, 1), 2), dtype=np.int64)
        k, done = ctypes.c_int32(0), ctypes.c_int32(0)
        st = self._lib.pa_bm_append_batch(self._h, _i64p(ids), _i32p(tok), ids.size,
                                          _i64p(slots), _i64p(pairs), ctypes.byref(k),
                                          ctypes.byref(done))
        if st < 0:
            err = PaError(st, "pa_bm_append_batch")
            err.done = done.value
            raise err
        return slots, pairs[:k.value].copy()

    def fork(self, parent: int, child: int):
        _check(self._lib.pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def free_seq(self, seq_id: int):
        _check(self._lib.pa_bm_free(self._h, int(seq_id)), "pa_bm_free")

    def slots(self, seq_id: int, first: int, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.int64)
        _check(self._lib.pa_bm_slots(self._h, int(seq_id), int(first), int(count), _i64p(out)),
               "pa_bm_slots")
        return out

    def table(self, seq_id: int, width: int) -> np.ndarray:
        row = np.empty(width, dtype=np.int32)
        _check(self._lib.pa_bm_block_table(self._h, int(seq_id), _i32p(row), int(width)),
               "pa_bm_block_table")
        return row

    def tables(self, seq_ids, width: int):
        """(block_tables int32 [n, width], context_lens int32 [n]) for the kernels."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tab = np.empty((ids.size, width), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        _check(self._lib.pa_bm_tables(self._h, _i64p(ids), ids.size, _i32p(tab), int(width),
                                      _i32p(lens)), "pa_bm_tables")
        return tab, lens

    def seq_len(self, seq_id: int) -> int:
        return _check(self._lib.pa_bm_seq_len(self._h, int(seq_id)), "pa_bm_seq_len")

    def refcount(self, block: int) -> int:
        return _check(self._lib.pa_bm_refcount(self._h, int(block)), "pa_bm_refcount")

    def block_key(self, seq_id: int, j: int) -> int:
        k = ctypes.c_uint64()
        _check(self._lib.pa_bm_block_key(self._h, int(seq_id), int(j), ctypes.byref(k)),
               "pa_bm_block_key")
        return k.value

    def stats(self):
        f, e, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(self._lib.pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(e),
                                     ctypes.byref(c)), "pa_bm_stats")
        return f.value, e.value, c.value

    def evictable(self):
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = _check(self._lib.pa_bm_evictable(self._h, _i32p(out), out.size), "pa_bm_evictable")
        return out[:n].tolist()

    def set_host_blocks(self, n: int):
        _check(self._lib.pa_bm_set_host_blocks(self._h, int(n)), "pa_bm_set_host_blocks")

    def _swap(self, fn, seq_id, where):
        cap = self.num_blocks
        pairs = np.empty((cap, 2), dtype=np.int64)
        n = _check(fn(self._h, int(seq_id), _i64p(pairs), cap), where)
        return pairs[:n].copy()

    def swap_out(self, seq_id: int) -> np.ndarray:
        """(device block, host block) pairs int64 [nb, 2] for pa_block_swap."""
        return self._swap(self._lib.pa_bm_swap_out, seq_id, "pa_bm_swap_out")

    def swap_in(self, seq_id: int) -> np.ndarray:
        """(host block, device block) pairs int64 [nb, 2] for pa_block_swap."""
        return self._swap(self._lib.pa_bm_swap_in, seq_id, "pa_bm_swap_in")

    def host_free(self) -> int:
        return _check(self._lib.pa_bm_host_free(self._h), "pa_bm_host_free")
