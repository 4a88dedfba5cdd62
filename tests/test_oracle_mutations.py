"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin fails.

Each mutation replaces one oracle function with a wrong variant for the duration of
the test; the pin suite must raise for every one of them, otherwise the pins would not
be able to tell a broken oracle from a correct one.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.cache_ops as cops
import oracle.block_manager as obm
import oracle.prefill as pf
import oracle.quantize as qz
import oracle.storage as st
from pins import ALL_PINS


def _fails(pins=ALL_PINS):
    failed = []
    for p in pins:
        try:
            p()
        except Exception as e:          # AssertionError, or a shape error the mistake causes
            failed.append((p.__name__, type(e).__name__))
    return failed


def _interleaved_gqa(h, group):
    return h % 2                        # kv heads interleaved instead of contiguous groups


def _no_truncation(pool, table_row, L, block_size, num_blocks):
    nb = (L + block_size - 1) // block_size
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    return pool[ids].reshape((nb * block_size,) + pool.shape[2:])   # attends padded slots


def _shifted_table(pool, table_row, L, block_size, num_blocks):
    nb = (L + block_size - 1) // block_size
    ids = np.asarray(np.roll(table_row[:nb], 1), dtype=np.int64)   # logical j -> table[j-1]
    return pool[ids].reshape((nb * block_size,) + pool.shape[2:])[:L]


def _unnormalised(qv, K, V, scale):
    s = scale * (K @ qv)
    p = np.exp(s - s.max())
    return p @ V, p


def _scale_squared(qv, K, V, scale):
    s = scale * scale * (K @ qv)
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ V, p


def _linear_weights(qv, K, V, scale):
    s = scale * (K @ qv)
    p = s - s.min() + 1e-3
    p = p / p.sum()
    return p @ V, p


def _bias8_table():
    t = np.empty(256)
    for code in range(256):
        sign = -1.0 if code >> 7 else 1.0
        e, m = (code >> 3) & 15, code & 7
        t[code] = np.nan if (e == 15 and m == 7) else (
            sign * m / 8 * 2.0 ** -7 if e == 0 else sign * (1 + m / 8) * 2.0 ** (e - 8))
    return t


def _bf16_low_half(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)).view(np.float32).astype(np.float64)


def _write_swapped(pool, new, slot_mapping):
    out = pool.copy()
    for t, s in enumerate(slot_mapping):
        if s >= 0:
            out[s % pool.shape[0], (s // pool.shape[0]) % pool.shape[1]] = new[t]
    return out


def _copy_reversed(pool, pairs):
    out = pool.copy()
    for s, d in np.asarray(pairs).reshape(-1, 2):
        out[s] = pool[d]
    return out


_good_encode = qz.e4m3_encode


def _encode_ties_away(y):
    out = _good_encode(y)
    y = np.asarray(y, dtype=np.float64).reshape(-1)
    flat = out.reshape(-1).copy()
    t = oracle.e4m3_table()
    for i, v in enumerate(y):               # at a tie take the larger magnitude instead
        c = int(flat[i]) & 0x7F
        if 0 < c < 0x7E and not np.isnan(v) and abs(v) == (t[c] + t[c + 1]) / 2:
            flat[i] = (int(flat[i]) & 0x80) | (c + 1)
    return flat.reshape(out.shape)


def _encode_no_saturation(y):
    out = _good_encode(y)
    big = np.abs(np.asarray(y, dtype=np.float64)) > 448.0
    return np.where(big, np.uint8(0x7F), out).astype(np.uint8)


def _encode_sign_dropped(y):
    return _good_encode(np.abs(np.asarray(y, dtype=np.float64)))


def _quant_scale_multiplies(new, kind, scale):
    x = st.decode_storage(new, kind).astype(np.float32)
    return x * np.float32(scale)


def _positions_from_start(L, n):
    return np.arange(0, n)                  # query token i at position i, not L - n + i


_good_attend = att.attend


def _prefill_no_causal_mask(q, query_start, k_pool, v_pool, block_tables, context_lens, scale,
                            *, q_kind, kv_kind, k_scale=1.0, v_scale=1.0):
    B = len(query_start) - 1
    out = np.zeros(q.shape, dtype=np.float64)
    G = q.shape[1] // k_pool.shape[2]
    N, bs = k_pool.shape[:2]
    for b in range(B):
        L = int(context_lens[b])
        K = st.decode_storage(att.gather_sequence(k_pool, block_tables[b], L, bs, N), kv_kind)
        V = st.decode_storage(att.gather_sequence(v_pool, block_tables[b], L, bs, N), kv_kind)
        for r in range(int(query_start[b]), int(query_start[b + 1])):
            qv = st.decode_storage(q[r], q_kind)
            for h in range(q.shape[1]):    # every token attends over all L positions
                out[r, h], _ = _good_attend(qv[h], K[:, h // G] * k_scale, V[:, h // G] * v_scale,
                                            scale)
    return out


def _positions_one_early(L, n):
    return np.arange(L - n, L) - 1          # the mask stops one position short


def _free_head_first(self, seq_id):
    s = self.seqs.pop(seq_id)
    for blk in s["blocks"]:                     # head first instead of tail first
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            (self.evictable if blk in self.block_key else self.free).append(blk)


_good_append = obm.BlockManager.append


def _append_no_cow(self, seq_id, token):
    s = self.seqs[seq_id]
    saved = self.ref[s["blocks"][-1]] if s["blocks"] else None
    if s["blocks"]:
        self.ref[s["blocks"][-1]] = 1           # pretend the last block is not shared
    try:
        return _good_append(self, seq_id, token)
    finally:
        if saved is not None and s["blocks"]:
            self.ref[s["blocks"][-1]] = max(self.ref[s["blocks"][-1]], saved)


_good_key = obm.block_key


def _key_unchained(prev, salt, tokens):
    return _good_key(0, salt, tokens)           # forgets the previous block's key


def _append_new_block_each_token(self, seq_id, token):
    s = self.seqs[seq_id]
    if self.available() < 1:
        raise obm.NoBlocks()
    s["blocks"].append(self._allocate())        # a block per token, full or not
    s["tokens"].append(token)
    return s["blocks"][-1] * self.bs, -1, -1


def _allocate_evicts_most_recent(self):
    if self.free:
        blk = self.free.pop(0)
    else:
        blk = self.evictable.pop()              # the most recently released
        del self.cache[self.block_key.pop(blk)]
        del self.block_tokens[blk]
    self.ref[blk] = 1
    return blk


def _swap_reversed(dst_pool, src_pool, pairs):
    out = np.array(dst_pool, copy=True)
    for s_, d in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        if 0 <= d < src_pool.shape[0] and 0 <= s_ < dst_pool.shape[0]:
            out[s_] = src_pool[d]                   # pair read as (dst, src)
    return out


_good_swap_out = obm.BlockManager.swap_out


def _swap_out_pairs_reversed(self, seq_id):
    return [(h, d) for d, h in _good_swap_out(self, seq_id)]


_good_head_scales = att.head_scales


def _head_scales_reversed(s, num_kv_heads):
    return _good_head_scales(s, num_kv_heads)[::-1].copy()    # head g gets scale[Hkv-1-g]


MUTATIONS = {
    "gqa_interleaved": (att, "kv_head_of", _interleaved_gqa),
    "no_length_mask": (att, "gather_sequence", _no_truncation),
    "table_off_by_one": (att, "gather_sequence", _shifted_table),
    "softmax_unnormalised": (att, "attend", _unnormalised),
    "scale_squared": (att, "attend", _scale_squared),
    "linear_not_exp": (att, "attend", _linear_weights),
    "e4m3_bias_8": (st, "e4m3_table", _bias8_table),
    "bf16_low_half": (st, "bf16_bits_to_f64", _bf16_low_half),
    "slot_index_swapped": (cops, "cache_write_ref", _write_swapped),
    "copy_direction_reversed": (cops, "block_copy_ref", _copy_reversed),
    "e4m3_ties_away_from_zero": (qz, "e4m3_encode", _encode_ties_away),
    "e4m3_no_saturation": (qz, "e4m3_encode", _encode_no_saturation),
    "e4m3_sign_dropped": (qz, "e4m3_encode", _encode_sign_dropped),
    "quant_scale_multiplies": (qz, "quant_inputs", _quant_scale_multiplies),
    "prefill_positions_from_start": (pf, "query_positions", _positions_from_start),
    "prefill_no_causal_mask": (pf, "prefill_ref", _prefill_no_causal_mask),
    "prefill_mask_one_short": (pf, "query_positions", _positions_one_early),
    "bm_release_head_first": (obm.BlockManager, "free_seq", _free_head_first),
    "bm_no_copy_on_write": (obm.BlockManager, "append", _append_no_cow),
    "bm_key_unchained": (obm, "block_key", _key_unchained),
    "bm_block_per_token": (obm.BlockManager, "append", _append_new_block_each_token),
    "bm_evicts_most_recent": (obm.BlockManager, "_allocate", _allocate_evicts_most_recent),
    "swap_pair_reversed": (cops, "block_swap_ref", _swap_reversed),
    "head_scales_reversed": (att, "head_scales", _head_scales_reversed),
    "bm_swap_out_pairs_reversed": (obm.BlockManager, "swap_out", _swap_out_pairs_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    # the package re-exports some names; patch those too so every caller sees the mistake
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    if mod is st and attr == "e4m3_table":
        monkeypatch.setattr(st, "_E4M3_CACHE", None)
    assert _fails(), f"no pin caught the planted mistake {name}"
