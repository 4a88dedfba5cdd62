"""Multi-token queries over the paged cache, fp64 reference (oracle; test infrastructure).

What is computed. A long prompt's prefill can be cut into chunks that run over several
steps next to decode tokens, and a prefix-cache hit skips the prefill of the cached
prefix so only the remaining tail is prefilled (LLM KV cache serving-engine article,
sections 3 "chunked prefill" and 4 "prefix caching"). Either way a step attends n new
query tokens of a sequence over that sequence's paged cache, which already holds their
own K/V rows (written by the slot write) after the earlier tokens'.

Reading taken here (the pages give no formula for it): sequence b has L = context_lens[b]
cached tokens, the last n = query_start[b+1] - query_start[b] of which are its new query
tokens; query token i (0 <= i < n) sits at position L - n + i and attends causally over
positions [0, L - n + i], with the same softmax, scale, GQA head mapping and fp8
dequantisation as the decode (a decode step is the case n = 1). The query rows of all
sequences are packed: q[query_start[b] + i] is sequence b's token i.
"""
from __future__ import annotations

import numpy as np

from .attention import attend, gather_sequence, head_scales, kv_head_of
from .storage import decode_storage


def query_positions(L: int, n: int) -> np.ndarray:
    """Positions of a sequence's n query tokens when it holds L tokens."""
    if not 0 <= n <= L:
        raise ValueError("a sequence's query tokens must be among its cached tokens")
    return np.arange(L - n, L)


def prefill_ref(q, query_start, k_pool, v_pool, block_tables, context_lens, scale, *,
                q_kind, kv_kind, k_scale=1.0, v_scale=1.0, rows=None):
    """Reference output, float64 [total query tokens, Hq, d].

    q: storage [Tq, Hq, d]; query_start: int [B + 1], non-decreasing, query_start[B] = Tq;
    k_pool/v_pool: storage [N, bs, Hkv, d]; block_tables: int [B, maxb];
    context_lens: int [B]; k_scale, v_scale: one number or one per kv head; rows: optional
    collection of query rows to compute (the others are left NaN), for sampled checks of
    large inputs."""
    Tq, Hq, d = q.shape
    N, bs, Hkv, dk = k_pool.shape
    if dk != d or v_pool.shape != k_pool.shape or Hq % Hkv:
        raise ValueError("shape mismatch between q and the pools")
    qs = np.asarray(query_start, dtype=np.int64)
    if qs[0] != 0 or qs[-1] != Tq or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must rise from 0 to the number of query rows")
    G = Hq // Hkv
    ks, vs = head_scales(k_scale, Hkv), head_scales(v_scale, Hkv)
    want = None if rows is None else set(int(r) for r in rows)
    out = np.zeros((Tq, Hq, d), dtype=np.float64)
    if want is not None:
        out[:] = np.nan
    for b in range(qs.size - 1):
        L, n = int(context_lens[b]), int(qs[b + 1] - qs[b])
        pos = query_positions(L, n)
        if n == 0 or (want is not None and not want & set(range(qs[b], qs[b + 1]))):
            continue
        K = decode_storage(gather_sequence(k_pool, block_tables[b], L, bs, N), kv_kind) * ks
        V = decode_storage(gather_sequence(v_pool, block_tables[b], L, bs, N), kv_kind) * vs
        qb = decode_storage(q[qs[b]:qs[b + 1]], q_kind)
        for i in range(n):
            if want is not None and int(qs[b]) + i not in want:
                continue
            last = int(pos[i]) + 1                     # causal: positions [0, pos]
            for h in range(Hq):
                g = kv_head_of(h, G)
                out[qs[b] + i, h], _ = attend(qb[i, h], K[:last, g, :], V[:last, g, :], scale)
    return out
