"""ctypes binding of libpa.so (argument marshalling only).

Tensors are torch tensors on the GPU; the binding checks device, contiguity and that
shapes agree, derives dtype codes, and passes data_ptr() values together with torch's
current HIP stream. Sizes follow include/paged_attention.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3

_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libpa.so")


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {pa_status_string(status)} ({status})")


class DecodeDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "block_size", "num_blocks",
        "max_blocks_per_seq", "q_dtype", "kv_dtype", "out_dtype", "partition_size")]


class PrefillDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_query_tokens", "num_q_heads", "num_kv_heads", "head_dim", "block_size",
        "num_blocks", "max_blocks_per_seq", "q_dtype", "kv_dtype", "out_dtype")]


def load_library():
    """Load libpa.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_367_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(DecodeDesc)
    lib.pa_abi_version.restype = I32
    lib.pa_abi_version.argtypes = []
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [I32]
    lib.pa_decode_max_chunks.restype = I32
    lib.pa_decode_max_chunks.argtypes = [D, I32]
    lib.pa_decode_workspace_bytes.restype = SZ
    lib.pa_decode_workspace_bytes.argtypes = [D, I32]
    lib.pa_decode.restype = I32
    lib.pa_decode.argtypes = [D, P, P, P, P, P, P, I32, F, F, F, P, SZ, P]
    lib.pa_decode_noalloc.restype = I32
    lib.pa_decode_noalloc.argtypes = [D, P, P, P, P, P, P, I32, F, F, F, P]
    lib.pa_decode_head_scales.restype = I32
    lib.pa_decode_head_scales.argtypes = [D, P, P, P, P, P, P, I32, F, P, P, P, SZ, P]
    lib.pa_prefill_head_scales.restype = I32
    lib.pa_prefill_head_scales.argtypes = [ctypes.POINTER(PrefillDesc), P, P, P, P, P, P, P,
                                           I32, F, P, P, P]
    lib.pa_cache_write_fp8_head_scales.restype = I32
    lib.pa_cache_write_fp8_head_scales.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                                   P, P, P]
    lib.pa_prefill.restype = I32
    lib.pa_prefill.argtypes = [ctypes.POINTER(PrefillDesc), P, P, P, P, P, P, P, I32, F, F, F, P]
    lib.pa_cache_write.restype = I32
    lib.pa_cache_write.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, P]
    lib.pa_cache_write_fp8.restype = I32
    lib.pa_cache_write_fp8.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, F, F, P]
    lib.pa_block_swap.restype = I32
    lib.pa_block_swap.argtypes = [P, P, I32, P, P, I32, P, I32, I32, I32, I32, I32, P]
    lib.pa_stream_read.restype = I32
    lib.pa_stream_read.argtypes = [P, SZ, P, I32, P]
    lib.pa_block_copy.restype = I32
    lib.pa_block_copy.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P]
    _LIB = lib
    return lib


def pa_abi_version() -> int:
    return load_library().pa_abi_version()


def pa_status_string(status: int) -> str:
    return load_library().pa_status_string(status).decode()


# ------------------------------------------------------------------ marshalling helpers

def dtype_code(t) -> int:
    import torch
    m = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16,
         torch.uint8: PA_FP8_E4M3, torch.float8_e4m3fn: PA_FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_desc(q, k_pool, block_tables, out=None, partition_size: int = 0) -> DecodeDesc:
    B, Hq, d = q.shape
    N, bs, Hkv, dk = k_pool.shape
    if dk != d:
        raise ValueError("head_dim of q and the pool differ")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [batch, max_blocks_per_seq]")
    return DecodeDesc(B, Hq, Hkv, d, bs, N, block_tables.shape[1], dtype_code(q),
                      dtype_code(k_pool), dtype_code(out if out is not None else q),
                      partition_size)


def pa_decode_max_chunks(desc: DecodeDesc, max_context_len: int) -> int:
    return load_library().pa_decode_max_chunks(ctypes.byref(desc), max_context_len)


def decode_workspace(desc: DecodeDesc, max_context_len: int, device="cuda"):
    """A workspace tensor for pa_decode (its contents need no initialisation: every call
    writes what it reads)."""
    import torch
    n = load_library().pa_decode_workspace_bytes(ctypes.byref(desc), int(max_context_len))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def pa_decode_workspace_bytes(desc: DecodeDesc, max_context_len: int) -> int:
    return load_library().pa_decode_workspace_bytes(ctypes.byref(desc), max_context_len)


def _head_scale_ptrs(k_scale, v_scale, num_kv_heads):
    """(per-tensor floats, per-head pointers): GPU float32 tensors of Hkv values select the
    per-head entry points."""
    import torch
    per_head = isinstance(k_scale, torch.Tensor) or isinstance(v_scale, torch.Tensor)
    if not per_head:
        return False, float(k_scale), float(v_scale), None, None
    for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or \
                t.shape != (num_kv_heads,):
            raise ValueError(f"{name}: per-head scales are float32 [num_kv_heads] GPU tensors")
    return True, 1.0, 1.0, _dev(k_scale, "k_scale"), _dev(v_scale, "v_scale")


def pa_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
              scale: float, k_scale=1.0, v_scale=1.0, workspace=None,
              partition_size: int = 0, stream=None):
    """Decode attention into `out` [B, Hq, d]. workspace: a uint8 GPU tensor of at least
    pa_decode_workspace_bytes() bytes, any contents (allocated here when None). k_scale / v_scale: floats, or float32 [Hkv] GPU tensors of per-head scales
    (pa_decode_head_scales)."""
    import torch
    lib = load_library()
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ in shape or dtype")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if context_lens.shape != (q.shape[0],):
        raise ValueError("context_lens must be [batch]")
    desc = make_desc(q, k_pool, block_tables, out, partition_size)
    need = lib.pa_decode_workspace_bytes(ctypes.byref(desc), int(max_context_len))
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    per_head, ks, vs, kp, vp = _head_scale_ptrs(k_scale, v_scale, k_pool.shape[2])
    common = (ctypes.byref(desc), _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
              _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables", torch.int32),
              _dev(context_lens, "context_lens", torch.int32), int(max_context_len),
              float(scale))
    if per_head:
        st = lib.pa_decode_head_scales(*common, kp, vp, ws_ptr, ws_bytes, _stream(stream))
    else:
        st = lib.pa_decode(*common, ks, vs, ws_ptr, ws_bytes, _stream(stream))
    if st != 0:
        raise PaError(st, "pa_decode_head_scales" if per_head else "pa_decode")
    return out


def pa_prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
               max_query_len: int, scale: float, k_scale=1.0, v_scale=1.0, stream=None):
    """Multi-token causal attention into `out` [Tq, Hq, d] for packed query rows q
    [Tq, Hq, d]; sequence b owns rows query_start[b] .. query_start[b+1] - 1 (int32
    [B + 1]), the last tokens of its context_lens[b] cached ones. k_scale / v_scale: floats,
    or float32 [Hkv] GPU tensors of per-head scales (pa_prefill_head_scales)."""
    import torch
    lib = load_library()
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ in shape or dtype")
    if out.shape != q.shape or q.dim() != 3:
        raise ValueError("q and out must be [num_query_tokens, num_q_heads, head_dim]")
    B = context_lens.shape[0]
    if query_start.shape != (B + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("query_start must be [batch + 1], block_tables [batch, max_blocks]")
    Tq, Hq, d = q.shape
    N, bs, Hkv, dk = k_pool.shape
    if dk != d:
        raise ValueError("head_dim of q and the pool differ")
    desc = PrefillDesc(B, Tq, Hq, Hkv, d, bs, N, block_tables.shape[1], dtype_code(q),
                       dtype_code(k_pool), dtype_code(out))
    per_head, ks, vs, kp, vp = _head_scale_ptrs(k_scale, v_scale, Hkv)
    common = (ctypes.byref(desc), _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"),
              _dev(v_pool, "v_pool"), _dev(block_tables, "block_tables", torch.int32),
              _dev(context_lens, "context_lens", torch.int32),
              _dev(query_start, "query_start", torch.int32), int(max_query_len), float(scale))
    if per_head:
        st = lib.pa_prefill_head_scales(*common, kp, vp, _stream(stream))
    else:
        st = lib.pa_prefill(*common, ks, vs, _stream(stream))
    if st != 0:
        raise PaError(st, "pa_prefill_head_scales" if per_head else "pa_prefill")
    return out


def pa_cache_write(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None):
    """Write new tokens' K/V [T, Hkv, d] into their slots (slot_mapping int64 [T])."""
    import torch
    lib = load_library()
    N, bs, Hkv, d = k_pool.shape
    T = slot_mapping.shape[0]
    if k_new.shape != (T, Hkv, d) or v_new.shape != (T, Hkv, d):
        raise ValueError("k_new / v_new must be [num_tokens, num_kv_heads, head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != v_pool.dtype or v_pool.shape != k_pool.shape:
        raise ValueError("new tokens and pools must share dtype and shape")
    st = lib.pa_cache_write(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                            _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int64),
                            T, Hkv, d, bs, N, dtype_code(k_pool), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_cache_write")


def pa_cache_write_fp8(k_pool, v_pool, k_new, v_new, slot_mapping, k_scale=1.0, v_scale=1.0,
                       stream=None):
    """Write new tokens' K/V [T, Hkv, d] (float32, float16 or bfloat16) into the slots of
    fp8 E4M3 pools (uint8 or float8_e4m3fn), quantising with dequantisation scales k_scale,
    v_scale: floats (per tensor) or float32 [Hkv] GPU tensors (per kv head)."""
    import torch
    lib = load_library()
    N, bs, Hkv, d = k_pool.shape
    T = slot_mapping.shape[0]
    if k_new.shape != (T, Hkv, d) or v_new.shape != (T, Hkv, d):
        raise ValueError("k_new / v_new must be [num_tokens, num_kv_heads, head_dim]")
    if v_pool.shape != k_pool.shape or dtype_code(k_pool) != PA_FP8_E4M3 or \
            dtype_code(v_pool) != PA_FP8_E4M3:
        raise ValueError("pools must be fp8 E4M3 bytes of the same shape")
    if v_new.dtype != k_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    per_head, ks, vs, kp, vp = _head_scale_ptrs(k_scale, v_scale, Hkv)
    common = (_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
              _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int64), T, Hkv, d,
              bs, N, dtype_code(k_new))
    if per_head:
        st = lib.pa_cache_write_fp8_head_scales(*common, kp, vp, _stream(stream))
    else:
        st = lib.pa_cache_write_fp8(*common, ks, vs, _stream(stream))
    if st != 0:
        raise PaError(st, "pa_cache_write_fp8_head_scales" if per_head else "pa_cache_write_fp8")


def pa_block_copy(k_pool, v_pool, src_dst_pairs, stream=None):
    """Copy whole blocks src -> dst in both pools (pairs int64 [P, 2])."""
    import torch
    lib = load_library()
    N, bs, Hkv, d = k_pool.shape
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [num_pairs, 2]")
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ in shape or dtype")
    st = lib.pa_block_copy(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                           _dev(src_dst_pairs, "src_dst_pairs", torch.int64),
                           src_dst_pairs.shape[0], Hkv, d, bs, N, dtype_code(k_pool),
                           _stream(stream))
    if st != 0:
        raise PaError(st, "pa_block_copy")


def _any_mem(t, name):
    """Pointer of a contiguous tensor on the GPU or in pinned host memory."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    return ctypes.c_void_p(t.data_ptr())


def pa_block_swap(dst_k, dst_v, src_k, src_v, src_dst_pairs, stream=None):
    """Copy whole blocks src -> dst between two pools (either may be pinned host memory);
    pairs int64 [P, 2] on the GPU or pinned."""
    import torch
    lib = load_library()
    if dst_k.shape[1:] != src_k.shape[1:] or dst_k.dtype != src_k.dtype:
        raise ValueError("the pools differ in block shape or dtype")
    if dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise ValueError("K and V pools differ in shape")
    if src_dst_pairs.dim() != 2 or src_dst_pairs.shape[1] != 2 or \
            src_dst_pairs.dtype != torch.int64:
        raise ValueError("src_dst_pairs must be int64 [num_pairs, 2]")
    N, bs, Hkv, d = dst_k.shape
    st = lib.pa_block_swap(_any_mem(dst_k, "dst_k"), _any_mem(dst_v, "dst_v"), N,
                           _any_mem(src_k, "src_k"), _any_mem(src_v, "src_v"), src_k.shape[0],
                           _any_mem(src_dst_pairs, "src_dst_pairs"), src_dst_pairs.shape[0],
                           Hkv, d, bs, dtype_code(dst_k), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_block_swap")


def pa_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len: int,
                      scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                      partition_size: int = 0, stream=None):
    """pa_decode with the library's static scratch as workspace: allocates nothing (neither
    here nor in the library). Calls overlapping on one GPU race (they share the scratch)."""
    import torch
    lib = load_library()
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool differ in shape or dtype")
    if out.shape != q.shape:
        raise ValueError("out must have the shape of q")
    if context_lens.shape != (q.shape[0],):
        raise ValueError("context_lens must be [batch]")
    desc = make_desc(q, k_pool, block_tables, out, partition_size)
    st = lib.pa_decode_noalloc(ctypes.byref(desc), _dev(out, "out"), _dev(q, "q"),
                               _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                               _dev(block_tables, "block_tables", torch.int32),
                               _dev(context_lens, "context_lens", torch.int32),
                               int(max_context_len), float(scale), float(k_scale),
                               float(v_scale), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_decode_noalloc")
    return out


def pa_stream_read(buf, sink, workgroups: int = 0, stream=None):
    """Read every byte of the GPU tensor `buf` once (a read-only bandwidth reference);
    `sink` is a GPU tensor of at least 4 bytes."""
    st = load_library().pa_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                       _dev(sink, "sink"), int(workgroups), _stream(stream))
    if st != 0:
        raise PaError(st, "pa_stream_read")
