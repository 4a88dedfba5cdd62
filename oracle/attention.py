"""Paged decode attention, fp64 reference (oracle; test infrastructure).

What is computed. One decode step: every sequence b has one query token q[b] with Hq
heads. Its keys and values live in fixed 16-token blocks anywhere in a physical pool
[num_blocks, block_size, kv_heads, head_dim]; its block table maps logical block j to
physical block table[b, j] (vLLM-PagedAttention与连续批处理技术拆解, sections 3.1-3.2;
the block-table example there maps logical 0, 1, 2 to physical 3, 11, 7).

The result is plain softmax attention over the sequence's first L = context_lens[b]
tokens. PagedAttention reaches exactly this value: its blockwise softmax with per-block
max and normaliser merged by rescaling is stated to be mathematically equivalent to
the global softmax (same page, section 3.3), and attention over scattered blocks gives
the same result as over a contiguous array (LLM KV cache serving-engine article,
section 2, "blocks and block table"). So the oracle is the definition itself, in the
order the sketch on "AI vLLM：PagedAttention不够用了之后" (section "PagedAttention 的计算
优化") gives: gather the sequence's blocks, scores = q K^T / sqrt(d), softmax, times V.

Readings where the pages are silent or garbled:
  * The sketch gathers whole blocks without truncating to the context length; the
    last block holds fewer than 16 tokens (serving-engine article, section 2), and
    the intelliparadigm article (section 5.1) warns to check the mask at block
    boundaries. Here only positions [0, L) are attended; other slots are never read.
  * GQA: query head h uses kv head h // (Hq / Hkv) (contiguous groups).
  * scale is an explicit argument (the workloads pass 1/sqrt(head_dim)).
  * L = 0 yields a zero output.
  * fp8 pools are dequantised as k_scale * E4M3(bits), v_scale * E4M3(bits).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .storage import decode_storage


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h when `group` query heads share one KV head."""
    return h // group


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, L: int, block_size: int,
                    num_blocks: int) -> np.ndarray:
    """Contiguous [L, Hkv, d] view of one sequence's tokens, still in storage encoding.

    Logical token t lives in physical block table_row[t // block_size] at slot
    t % block_size."""
    nb = (L + block_size - 1) // block_size
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if ids.size and (ids.min() < 0 or ids.max() >= num_blocks):
        raise ValueError("block table entry outside the pool")
    if np.unique(ids).size != ids.size:
        raise ValueError("block table row repeats a physical block")
    blocks = pool[ids]                                   # [nb, bs, Hkv, d]
    return blocks.reshape((nb * block_size,) + pool.shape[2:])[:L]


def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Textbook softmax attention of one query vector over K, V ([L, d] each, fp64).

    Returns (output [d], probabilities [L])."""
    s = scale * (K @ qv)                     # scores, [L]
    p = np.exp(s - s.max())                  # subtracting the max changes nothing exactly
    p = p / p.sum()
    return p @ V, p


def head_scales(s, num_kv_heads: int) -> np.ndarray:
    """A dequantisation scale per kv head, shaped [Hkv, 1] to multiply [..., Hkv, d]: one
    number for the whole tensor, or one per kv head (each head's codes times its own)."""
    a = np.asarray(s, dtype=np.float64).reshape(-1)
    if a.size == 1:
        a = np.full(num_kv_heads, a[0])
    if a.size != num_kv_heads:
        raise ValueError("one scale, or one per kv head")
    return a.reshape(num_kv_heads, 1)


def decode_ref(q, k_pool, v_pool, block_tables, context_lens, scale, *, q_kind, kv_kind,
               k_scale=1.0, v_scale=1.0, seqs: Optional[Iterable[int]] = None,
               return_probs: bool = False):
    """Reference decode output, float64 [len(seqs) or B, Hq, d].

    q: storage [B, Hq, d]; k_pool/v_pool: storage [N, bs, Hkv, d];
    block_tables: int [B, maxb] (-1 padding); context_lens: int [B].
    k_scale, v_scale: dequantisation scales, one number or one per kv head.
    seqs restricts the computation to a subset of sequences (in that order)."""
    B, Hq, d = q.shape
    N, bs, Hkv, dk = k_pool.shape
    if dk != d or v_pool.shape != k_pool.shape:
        raise ValueError("shape mismatch between q and the pools")
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    G = Hq // Hkv
    ks, vs = head_scales(k_scale, Hkv), head_scales(v_scale, Hkv)
    order = list(range(B)) if seqs is None else [int(b) for b in seqs]
    out = np.zeros((len(order), Hq, d), dtype=np.float64)
    probs = {}
    for i, b in enumerate(order):
        L = int(context_lens[b])
        if L <= 0:
            continue
        K = decode_storage(gather_sequence(k_pool, block_tables[b], L, bs, N), kv_kind) * ks
        V = decode_storage(gather_sequence(v_pool, block_tables[b], L, bs, N), kv_kind) * vs
        qb = decode_storage(q[b], q_kind)
        for h in range(Hq):
            g = kv_head_of(h, G)
            o, p = attend(qb[h], K[:, g, :], V[:, g, :], scale)
            out[i, h] = o
            if return_probs:
                probs[(b, h)] = p
    return (out, probs) if return_probs else out
