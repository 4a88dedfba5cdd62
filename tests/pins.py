"""Pins that tie the CPU oracle to things other than itself.

Each pin raises AssertionError when the oracle disagrees with a value the pages print,
a closed form, an invariant the pages state, a library routine, or brute force. They
are plain functions so that tests/test_oracle_mutations.py can re-run all of them
against an oracle with a planted mistake and check that some pin catches it.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
import workload as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ref(w, **kw):
    return oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale,
                             q_kind=w.q_dtype, kv_kind=w.kv_dtype, k_scale=w.k_scale,
                             v_scale=w.v_scale, **kw)


def _torch_tables():
    """Decoders built from torch's own dtype conversions (independent of oracle.storage)."""
    import torch
    e4m3 = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    bits16 = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    return {
        "fp8_e4m3": e4m3.to(torch.float64).numpy(),
        "bf16": bits16.view(torch.bfloat16).to(torch.float64).numpy(),
        "f16": bits16.view(torch.float16).to(torch.float64).numpy(),
    }


def _decode_lib(arr, kind, tabs):
    if kind == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if kind == "f16":
        return tabs["f16"][np.asarray(arr).view(np.uint16)]
    return tabs[kind][np.asarray(arr)]


def contiguous_cache(w, tabs=None):
    """D10-style contiguous per-request cache [B, maxL, Hkv, d] in float64, built slot by slot.

    Mirrors the pre-paging layout (one [max_seq_len, heads, head_dim] tensor per request)
    from the intelliparadigm article, section 2.1. Decoding uses torch's conversions."""
    tabs = tabs or _torch_tables()
    B, maxL = w.batch, max(1, w.max_context_len)
    Kc = np.zeros((B, maxL, w.num_kv_heads, w.head_dim))
    Vc = np.zeros_like(Kc)
    for b in range(B):
        for t in range(int(w.context_lens[b])):
            p = int(w.block_tables[b, t // w.block_size])
            Kc[b, t] = _decode_lib(w.k_pool[p, t % w.block_size], w.kv_dtype, tabs) * w.k_scale
            Vc[b, t] = _decode_lib(w.v_pool[p, t % w.block_size], w.kv_dtype, tabs) * w.v_scale
    return Kc, Vc


# ------------------------------------------------------------------ printed values

def pin_kv_formula():
    g = json.load(open(os.path.join(GOLDEN, "kv_formula.json")))
    for c in g["cases"]:
        per = oracle.kv_bytes_per_token(c["layers"], c["kv_heads"], c["head_dim"], c["bytes"])
        assert per == c["per_token_bytes"], (c["model"], per)
        req = oracle.kv_bytes_per_request(c["request_tokens"], c["layers"], c["kv_heads"],
                                          c["head_dim"], c["bytes"])
        assert req == c["request_bytes"], (c["model"], req)


def pin_block_table_example():
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bs, N = g["block_size"], g["pool_blocks"]
    pool = np.zeros((N, bs, 1, 1), dtype=np.float32)
    for blk in range(N):
        for s in range(bs):
            pool[blk, s, 0, 0] = 100 * blk + s
    table = np.array(g["table"], dtype=np.int32)
    L = max(t for t, _, _ in g["probe_tokens"]) + 1
    seq = oracle.gather_sequence(pool, table, L, bs, N)
    assert seq.shape[0] == L
    for t, blk, slot in g["probe_tokens"]:
        assert seq[t, 0, 0] == 100 * blk + slot, (t, seq[t, 0, 0])


# ------------------------------------------------------------------ paging invariants

def _small(kv="bf16", G=4, Hkv=2, d=64, lens=(1, 16, 17, 40, 95), seed=0, **kw):
    return wl.custom(batch=len(lens), num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                     kv_dtype=kv, context_lens=list(lens), seed=seed, **kw)


def pin_permutation_invariance():
    """Moving physical blocks (and rewriting the tables) leaves the output bitwise equal."""
    w = _small()
    base = _ref(w)
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    t2 = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w.k_pool, w.v_pool, w.block_tables = k2, v2, t2
    assert np.array_equal(_ref(w), base)


def pin_contiguous_equality():
    """Paged attention equals attention over the contiguous pre-paging cache (bitwise)."""
    w = _small(kv="f16", G=2)
    Kc, Vc = contiguous_cache(w)
    out = _ref(w)
    tabs = _torch_tables()
    for b in range(w.batch):
        L = int(w.context_lens[b])
        qb = _decode_lib(w.q[b], w.q_dtype, tabs)
        for h in range(w.num_q_heads):
            g = h // w.group
            o, _ = oracle.attend(qb[h], Kc[b, :L, g], Vc[b, :L, g], w.scale)
            assert np.array_equal(o, out[b, h]), (b, h)


def pin_nan_poison():
    """NaN in every slot outside [0, L) changes nothing (masking by selection)."""
    clean = _small(lens=(3, 16, 33, 47))
    dirty = wl.poison_unused(_small(lens=(3, 16, 33, 47)))
    a, b = _ref(clean), _ref(dirty)
    assert np.isfinite(b).all()
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ softmax closed forms

def pin_rows_sum_to_one():
    w = _small()
    _, probs = _ref(w, return_probs=True)
    for (b, h), p in probs.items():
        assert p.shape == (int(w.context_lens[b]),)
        assert (p >= 0).all()
        assert abs(p.sum() - 1.0) <= 1e-12


def pin_single_token():
    """L = 1: the only probability is 1, so the output is that token's V row exactly."""
    w = _small(kv="f32", lens=(1, 1, 1))
    out = _ref(w)
    tabs = _torch_tables()
    for b in range(w.batch):
        v = _decode_lib(w.v_pool[w.block_tables[b, 0], 0], w.kv_dtype, tabs)
        for h in range(w.num_q_heads):
            assert np.array_equal(out[b, h], v[h // w.group]), (b, h)


def pin_constant_keys():
    """Equal keys for every token: uniform weights, output = mean of the V rows."""
    w = _small(kv="f32", lens=(5, 16, 29))
    Kc, Vc = contiguous_cache(w)
    rng = np.random.default_rng(1)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        row = rng.standard_normal((w.num_kv_heads, w.head_dim)).astype(np.float32)
        for t in range(L):
            w.k_pool[w.block_tables[b, t // 16], t % 16] = row
    out = _ref(w)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        for h in range(w.num_q_heads):
            mean = Vc[b, :L, h // w.group].mean(axis=0)
            assert np.max(np.abs(out[b, h] - mean)) <= 1e-12


def pin_zero_query():
    w = _small(kv="bf16", lens=(7, 40))
    w.q[:] = 0
    Kc, Vc = contiguous_cache(w)
    out = _ref(w)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        for h in range(w.num_q_heads):
            assert np.max(np.abs(out[b, h] - Vc[b, :L, h // w.group].mean(axis=0))) <= 1e-12


def pin_two_tokens():
    """L = 2: out = sigmoid(s0 - s1) v0 + sigmoid(s1 - s0) v1."""
    w = _small(kv="f32", lens=(2, 2), G=2)
    Kc, Vc = contiguous_cache(w)
    out = _ref(w)
    q = w.q.astype(np.float64)
    for b in range(w.batch):
        for h in range(w.num_q_heads):
            g = h // w.group
            s0 = w.scale * math.fsum(q[b, h] * Kc[b, 0, g])
            s1 = w.scale * math.fsum(q[b, h] * Kc[b, 1, g])
            a0 = 1.0 / (1.0 + math.exp(s1 - s0))
            a1 = 1.0 / (1.0 + math.exp(s0 - s1))
            exp = a0 * Vc[b, 0, g] + a1 * Vc[b, 1, g]
            assert np.max(np.abs(out[b, h] - exp)) <= 1e-12


def pin_blockwise_merge():
    """Blockwise softmax with per-block (m, l) merged by rescaling equals the global softmax.

    Block statistics and the rescale merge as described in vLLM-PagedAttention与连续批处理
    技术拆解, section 3.3, applied at 16-token blocks and again across 3-block partitions."""
    w = _small(kv="bf16", lens=(16, 17, 100, 250), d=64)
    Kc, Vc = contiguous_cache(w)
    out = _ref(w)
    tabs = _torch_tables()
    bs, part = w.block_size, 3
    for b in range(w.batch):
        L = int(w.context_lens[b])
        qb = _decode_lib(w.q[b], w.q_dtype, tabs)
        for h in range(w.num_q_heads):
            g = h // w.group
            partials = []
            for p0 in range(0, L, bs * part):
                m, l, acc = -np.inf, 0.0, np.zeros(w.head_dim)
                for j0 in range(p0, min(L, p0 + bs * part), bs):
                    K = Kc[b, j0:min(L, j0 + bs), g]
                    V = Vc[b, j0:min(L, j0 + bs), g]
                    s = w.scale * (K @ qb[h])
                    m_blk = s.max()
                    m_new = max(m, m_blk)
                    e = np.exp(s - m_new)
                    alpha = math.exp(m - m_new) if m > -np.inf else 0.0
                    l = l * alpha + e.sum()
                    acc = acc * alpha + e @ V
                    m = m_new
                partials.append((m, l, acc))
            M = max(p[0] for p in partials)
            Ls = sum(p[1] * math.exp(p[0] - M) for p in partials)
            O = sum(p[2] * math.exp(p[0] - M) for p in partials) / Ls
            assert np.max(np.abs(O - out[b, h])) <= 1e-12, (b, h)


# ------------------------------------------------------------------ brute force & library

def _brute(w, tabs):
    out = np.zeros((w.batch, w.num_q_heads, w.head_dim))
    for b in range(w.batch):
        L = int(w.context_lens[b])
        qb = _decode_lib(w.q[b], w.q_dtype, tabs).tolist()
        for h in range(w.num_q_heads):
            g = h // w.group
            ks, vs = [], []
            for t in range(L):
                blk, slot = int(w.block_tables[b][t // 16]), t % 16
                ks.append([w.k_scale * x for x in
                           _decode_lib(w.k_pool[blk][slot][g], w.kv_dtype, tabs).tolist()])
                vs.append([w.v_scale * x for x in
                           _decode_lib(w.v_pool[blk][slot][g], w.kv_dtype, tabs).tolist()])
            s = [w.scale * math.fsum(qb[h][i] * k[i] for i in range(w.head_dim)) for k in ks]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = math.fsum(e)
            for i in range(w.head_dim):
                out[b, h, i] = math.fsum(e[t] * vs[t][i] for t in range(L)) / z
    return out


def pin_brute_force_scalar():
    tabs = _torch_tables()
    for w in (wl.make(1), _small(kv="fp8_e4m3", lens=(9, 33), d=64, Hkv=1, G=2)):
        if w.kv_dtype == "fp8_e4m3":
            w.k_scale, w.v_scale = 0.0123, 0.0456   # distinct scales catch swapped ones
        ref = _ref(w)
        bf = _brute(w, tabs)
        assert np.max(np.abs(ref - bf)) <= 1e-12, w.name


def pin_block_removed_from_table():
    """Dropping a full block from a sequence's table (and 16 from its length) gives the
    attention over the sequence's other tokens, by brute force: the expected value the GPU
    tests use for a block id outside the pool, whose tokens the kernels leave out."""
    import dataclasses
    tabs = _torch_tables()
    w = _small(kv="bf16", G=2, Hkv=1, d=64, lens=(40, 33))
    j = 1                                               # the middle block of sequence 0
    t2 = w.block_tables.copy()
    t2[0, :2] = [w.block_tables[0, 0], w.block_tables[0, 2]]
    t2[0, 2] = -1
    red = dataclasses.replace(w, block_tables=t2,
                              context_lens=np.array([24, 33], dtype=np.int32))
    got = _ref(red)
    # brute force over the original table, skipping tokens 16 .. 31 of sequence 0
    keep = [t for t in range(40) if t // 16 != j]
    qb = _decode_lib(w.q[0], w.q_dtype, tabs).tolist()
    for h in range(w.num_q_heads):
        ks = [_decode_lib(w.k_pool[w.block_tables[0][t // 16]][t % 16][0], w.kv_dtype,
                          tabs).tolist() for t in keep]
        vs = [_decode_lib(w.v_pool[w.block_tables[0][t // 16]][t % 16][0], w.kv_dtype,
                          tabs).tolist() for t in keep]
        s = [w.scale * math.fsum(qb[h][i] * k[i] for i in range(w.head_dim)) for k in ks]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = math.fsum(e)
        want = [math.fsum(e[t] * vs[t][i] for t in range(len(keep))) / z
                for i in range(w.head_dim)]
        assert np.max(np.abs(got[0, h] - np.array(want))) <= 1e-12
    assert np.array_equal(got[1], _ref(w)[1])          # the other sequence is untouched


def pin_sdpa_library():
    """torch's scaled_dot_product_attention in float64 on the contiguous cache."""
    import torch
    for w in (wl.make(1), _small(kv="bf16", G=4, Hkv=2, lens=(1, 30, 77))):
        Kc, Vc = contiguous_cache(w)
        out = _ref(w)
        tabs = _torch_tables()
        for b in range(w.batch):
            L = int(w.context_lens[b])
            q = torch.from_numpy(_decode_lib(w.q[b], w.q_dtype, tabs))[None, :, None, :]
            k = torch.from_numpy(Kc[b, :L]).permute(1, 0, 2).repeat_interleave(w.group, 0)[None]
            v = torch.from_numpy(Vc[b, :L]).permute(1, 0, 2).repeat_interleave(w.group, 0)[None]
            o = torch.nn.functional.scaled_dot_product_attention(
                q.contiguous(), k.contiguous(), v.contiguous(), scale=w.scale)
            assert np.max(np.abs(o[0, :, 0, :].numpy() - out[b])) <= 1e-12, (w.name, b)


def pin_gqa_equals_repeated_mha():
    """GQA with group G equals MHA whose kv heads are each repeated G times in order."""
    w = _small(kv="bf16", G=4, Hkv=2)
    ref = _ref(w)
    G = w.group
    w.k_pool = np.repeat(w.k_pool, G, axis=2)
    w.v_pool = np.repeat(w.v_pool, G, axis=2)
    w.num_kv_heads *= G
    assert np.array_equal(_ref(w), ref)


# ------------------------------------------------------------------ storage decoding

def pin_storage_vs_torch():
    tabs = _torch_tables()
    codes8 = np.arange(256, dtype=np.uint8)
    a, b = oracle.decode_storage(codes8, "fp8_e4m3"), tabs["fp8_e4m3"]
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
    assert oracle.e4m3_table()[0x7E] == 448.0 and oracle.e4m3_table()[0x01] == 2.0 ** -9
    codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for kind, arr in (("bf16", codes16), ("f16", codes16.view(np.float16))):
        a, b = oracle.decode_storage(arr, kind), tabs[kind]
        assert np.array_equal(np.isnan(a), np.isnan(b)), kind
        assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)]), kind


# ------------------------------------------------------------------ cache write / copy

def pin_cache_write_closed_form():
    w = wl.make(1)
    slots = w.slot_mapping.copy()
    slots[1] = -1                                   # skipped entry
    out = oracle.cache_write_ref(w.k_pool, w.k_new, slots)
    touched = np.zeros(w.k_pool.shape[:2], dtype=bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(out[s // 16, s % 16].view(np.uint32), w.k_new[t].view(np.uint32))
        touched[s // 16, s % 16] = True
    assert np.array_equal(out[~touched].view(np.uint32), w.k_pool[~touched].view(np.uint32))


def pin_block_copy_closed_form():
    w = _small(kv="bf16")
    pairs = np.array([[w.block_tables[0, 0], w.num_blocks - 1],
                      [w.block_tables[2, 1], w.num_blocks - 2]], dtype=np.int64)
    out = oracle.block_copy_ref(w.k_pool, pairs)
    for s, d in pairs:
        assert np.array_equal(out[d], w.k_pool[s])
    keep = np.setdiff1d(np.arange(w.num_blocks), pairs[:, 1])
    assert np.array_equal(out[keep], w.k_pool[keep])


def pin_cow_isolation():
    """Copy-on-write keeps the shared prefix read-only and isolates every sample's tail."""
    w = wl.make(4, batch=2)
    k = oracle.block_copy_ref(w.k_pool, w.copy_pairs)
    v = oracle.block_copy_ref(w.v_pool, w.copy_pairs)
    fill = w.notes["partial_fill"]
    for s, d in w.copy_pairs:                  # copies equal the original before any tail write
        assert np.array_equal(k[d], w.k_pool[s]) and np.array_equal(v[d], w.v_pool[s])
    k2 = oracle.cache_write_ref(k, w.k_new, w.slot_mapping)
    v2 = oracle.cache_write_ref(v, w.v_new, w.slot_mapping)
    nfull = w.notes["shared_full_blocks"]
    shared = np.unique(w.block_tables[:, :nfull])
    assert np.array_equal(k2[shared], w.k_pool[shared]) and np.array_equal(v2[shared], w.v_pool[shared])
    # every sample's partial block keeps the prompt's first `fill` tokens, then its own tail
    S = w.notes["samples"]
    for b in range(w.batch):
        blk = w.block_tables[b, nfull]
        src = w.block_tables[(b // S) * S + S - 1, nfull]   # last sample keeps the original
        assert np.array_equal(k2[blk, :fill], w.k_pool[src, :fill])
        t0 = b * w.notes["tail"]
        assert np.array_equal(k2[blk, fill:], w.k_new[t0:t0 + 16 - fill])
    # every table entry is distinct within a row; only the full prefix blocks are shared
    for b in range(w.batch):
        assert np.unique(w.block_tables[b]).size == w.block_tables.shape[1]
    counts = np.bincount(w.block_tables.reshape(-1), minlength=w.num_blocks)
    assert set(np.unique(counts[counts > 0])) <= {1, S}
    assert (counts == S).sum() == nfull * w.notes["prompts"]


# ---- fp8 E4M3 quantisation on the slot write (oracle.quantize) ----------------------

def _e4m3_finite_codes():
    t = oracle.e4m3_table()
    return np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)


def pin_e4m3_round_trip():
    """Every finite code point encodes back to itself (254 of them: 0x7F, 0xFF are NaN)."""
    import oracle.quantize as qz
    codes = _e4m3_finite_codes()
    assert len(codes) == 254
    assert np.array_equal(qz.e4m3_encode(oracle.e4m3_table()[codes]), codes)


def pin_e4m3_midpoints_to_even():
    """Round to nearest, ties to the even mantissa, at every midpoint of both signs."""
    import oracle.quantize as qz
    t = oracle.e4m3_table()
    for sign in (0x00, 0x80):
        for c in range(0x7E):
            lo, hi = t[sign | c], t[sign | (c + 1)]
            mid = (lo + hi) / 2
            even = c if c % 2 == 0 else c + 1
            got = qz.e4m3_encode(np.array([mid - (hi - lo) / 16, mid, mid + (hi - lo) / 16]))
            assert got.tolist() == [sign | c, sign | even, sign | (c + 1)], (hex(sign | c), mid)


def pin_e4m3_saturation_nan_zero():
    """Saturation to +-448 (infinities included), NaN -> 0x7F, signed zeros kept."""
    import oracle.quantize as qz
    y = np.array([448.0, 463.9, 464.0, 1e30, np.inf, -1000.0, -np.inf, np.nan, 0.0, -0.0,
                  2.0 ** -10, 2.0 ** -10 * 1.001, -(2.0 ** -11)])
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x00, 0x80, 0x00, 0x01, 0x80]
    assert qz.e4m3_encode(y).tolist() == want


def pin_e4m3_vs_torch_cast():
    """torch's float8_e4m3fn cast (the same format, a library routine) on in-range values."""
    import torch
    import oracle.quantize as qz
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.normal(0, 1, 8000), rng.normal(0, 60, 8000),
                        rng.uniform(-447.0, 447.0, 8000), rng.normal(0, 0.01, 8000)])
    y = y.astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(qz.e4m3_encode(y), ref)


def pin_quant_power_of_two_scale():
    """With a power-of-two scale s, x = v * s for every E4M3 value v encodes to v's code
    (the scale divides, exactly), from fp32, fp16 and bf16 sources."""
    import oracle.quantize as qz
    t = oracle.e4m3_table()
    codes = np.array([c for c in _e4m3_finite_codes() if abs(t[c]) >= 2.0 ** -6], dtype=np.uint8)
    x = t[codes] * 8.0
    for kind, store in (("f32", x.astype(np.float32)), ("f16", x.astype(np.float16)),
                        ("bf16", (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))):
        y = qz.quant_inputs(store, kind, 8.0)
        assert y.dtype == np.float32
        assert np.array_equal(qz.e4m3_encode(y), codes), kind


def pin_cache_write_fp8_closed_form():
    """Slot s receives the codes of its new row (block s // 16, row s % 16); -1 skips;
    decoding the codes gives new / scale to within half a code spacing."""
    import oracle.quantize as qz
    rng = np.random.default_rng(1)
    pool = rng.integers(0, 256, size=(4, 16, 2, 8), dtype=np.uint8)
    new = rng.normal(0, 3, size=(3, 2, 8)).astype(np.float32)
    out = qz.cache_write_fp8_ref(pool, new, "f32", 0.5, np.array([5, -1, 63]))
    touched = np.zeros(out.shape[:2], dtype=bool)
    touched[0, 5] = touched[3, 15] = True
    assert np.array_equal(out[~touched], pool[~touched])
    for (blk, row), t in (((0, 5), 0), ((3, 15), 2)):
        dec = oracle.decode_storage(out[blk, row], "fp8_e4m3")
        target = np.clip(new[t].astype(np.float64) / 0.5, -448, 448)
        spacing = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(target), 2.0 ** -6))) - 3),
                             2.0 ** -9)
        assert np.all(np.abs(dec - target) <= spacing / 2 + 1e-12)


# ---- multi-token queries over the paged cache (oracle.prefill) ----------------------

def _prefill_case(n_per_seq, kv="bf16", G=4, Hkv=2, d=64, seed=3):
    """A small paged workload with n_per_seq[b] query tokens at the end of sequence b."""
    rng = np.random.default_rng(seed)
    w = wl.make(3, batch=len(n_per_seq), len_range=(20, 90), seed_offset=seed)
    # the workload's lengths and block tables, with pools of Hkv heads of d dims
    N = w.num_blocks
    k = wl._normal_storage(rng, (N, 16, Hkv, d), kv)
    v = wl._normal_storage(rng, (N, 16, Hkv, d), kv)
    qs = np.concatenate([[0], np.cumsum(n_per_seq)]).astype(np.int64)
    q = wl._normal_storage(rng, (int(qs[-1]), G * Hkv, d), "bf16")
    return dict(q=q, qs=qs, k=k, v=v, tables=w.block_tables, lens=w.context_lens,
                scale=1.0 / np.sqrt(d), kv=kv)


def _prefill(c, **kw):
    import oracle.prefill as pf
    args = dict(c, **kw)
    return pf.prefill_ref(args["q"], args["qs"], args["k"], args["v"], args["tables"],
                          args["lens"], args["scale"], q_kind="bf16", kv_kind=args["kv"],
                          rows=args.get("rows"))


def pin_prefill_one_token_is_decode():
    """One query token per sequence is exactly a decode step (same bits)."""
    c = _prefill_case([1, 1, 1, 1])
    got = _prefill(c)
    ref = oracle.decode_ref(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["scale"],
                            q_kind="bf16", kv_kind="bf16")
    assert np.array_equal(got, ref)


def pin_prefill_causality():
    """A token never sees later positions: changing K and V at position p leaves every
    query token before p unchanged (bitwise) and changes the tokens at or after it."""
    c = _prefill_case([9, 3])
    base = _prefill(c)
    b, L, n = 0, int(c["lens"][0]), 9
    p = L - 4                                       # among the query tokens: i = n - 4
    k2, v2 = c["k"].copy(), c["v"].copy()
    blk, row = c["tables"][b][p // 16], p % 16
    k2[blk, row] = np.uint16(0x4040)                         # bf16 3.0: a large change
    v2[blk, row] = np.uint16(0xC000)                         # bf16 -2.0
    pert = _prefill(c, k=k2, v=v2)
    i_p = p - (L - n)
    assert np.array_equal(pert[:i_p], base[:i_p])
    assert np.all(np.abs(pert[i_p:n] - base[i_p:n]).max(axis=(1, 2)) > 1e-6)
    assert np.array_equal(pert[n:], base[n:])                  # the other sequence


def pin_prefill_vs_sdpa():
    """torch's scaled_dot_product_attention in float64 with an explicit end-aligned
    causal mask on the contiguous K/V (a library routine with its own masking)."""
    import torch
    c = _prefill_case([6, 2, 11], G=2, Hkv=2)
    got = _prefill(c)
    G = c["q"].shape[1] // c["k"].shape[2]
    for b in range(3):
        L, n = int(c["lens"][b]), int(c["qs"][b + 1] - c["qs"][b])
        K = oracle.decode_storage(oracle.gather_sequence(c["k"], c["tables"][b], L, 16,
                                                         c["k"].shape[0]), "bf16")
        V = oracle.decode_storage(oracle.gather_sequence(c["v"], c["tables"][b], L, 16,
                                                         c["v"].shape[0]), "bf16")
        Q = oracle.decode_storage(c["q"][c["qs"][b]:c["qs"][b + 1]], "bf16")
        Kh = np.repeat(K, G, axis=1).transpose(1, 0, 2)[None]      # [1, Hq, L, d]
        Vh = np.repeat(V, G, axis=1).transpose(1, 0, 2)[None]
        Qh = Q.transpose(1, 0, 2)[None]                              # [1, Hq, n, d]
        mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Qh), torch.from_numpy(Kh), torch.from_numpy(Vh),
            attn_mask=torch.from_numpy(mask), scale=c["scale"]).numpy()[0].transpose(1, 0, 2)
        assert np.abs(got[c["qs"][b]:c["qs"][b + 1]] - ref).max() < 1e-12


def pin_prefill_full_prompt_first_token():
    """With every cached token a query token (n = L), token 0 attends to itself only,
    so its output is its own V row exactly."""
    c = _prefill_case([1])
    L = int(c["lens"][0])
    c["qs"] = np.array([0, L])
    rng = np.random.default_rng(9)
    c["q"] = wl._normal_storage(rng, (L, c["q"].shape[1], c["q"].shape[2]), "bf16")
    got = _prefill(c)
    V0 = oracle.decode_storage(c["v"][c["tables"][0][0], 0], "bf16")      # [Hkv, d]
    G = c["q"].shape[1] // c["v"].shape[2]
    assert np.array_equal(got[0], np.repeat(V0, G, axis=0))


def pin_prefill_sequences_independent():
    """Sequence b's outputs depend on its own query rows only."""
    c = _prefill_case([4, 5, 2])
    base = _prefill(c)
    q2 = c["q"].copy()
    q2[4:9] = q2[4:9] ^ np.uint16(0x0100)                       # sequence 1's rows
    pert = _prefill(c, q=q2)
    assert np.array_equal(pert[:4], base[:4]) and np.array_equal(pert[9:], base[9:])
    assert not np.array_equal(pert[4:9], base[4:9])




def pin_prefill_sampled_rows_equal_full():
    """Computing a subset of rows gives those rows of the full result, and NaN elsewhere."""
    c = _prefill_case([3, 9], kv="bf16", G=2, Hkv=2, d=64, seed=21)
    full = _prefill(c)
    rows = [0, 4, 11]
    part = _prefill(c, rows=rows)
    assert np.array_equal(part[rows], full[rows])
    others = [r for r in range(full.shape[0]) if r not in rows]
    assert np.isnan(part[others]).all()


# ----------------------------------------------------------------------------- block manager

def _bm(n, bs=16, prefix=True):
    import oracle.block_manager as obm
    return obm.BlockManager(n, bs, prefix)


def pin_bm_fnv1a64_published_vectors():
    """FNV-1a 64-bit against the published test vectors of its definition."""
    import oracle.block_manager as obm
    assert obm.fnv1a64(b"") == 0xCBF29CE484222325
    assert obm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert obm.fnv1a64(b"foobar") == 0x85944171F73967E8


def pin_bm_table_example():
    """The pages' table (logical 0 -> 3, 1 -> 11, 2 -> 7): a sequence that grows through
    three blocks takes them from the free list in order, and its token positions map to
    slots through the table (the golden probes)."""
    g = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bs, want = g["block_size"], g["table"]
    m = _bm(g["pool_blocks"], bs, prefix=False)
    for i in range(g["pool_blocks"]):                 # one block each: sequence i holds block i
        m.add(i, [i] * bs)
    for blk in want:                                  # free list becomes 3, 11, 7
        m.free_seq(blk)
    m.add(100, [])
    slots = [m.append(100, 7)[0] for _ in range(41)]
    assert m.table(100, 3) == want
    for pos, blk, off in g["probe_tokens"]:
        assert slots[pos] == blk * bs + off


def pin_bm_waste_below_one_block():
    """The only waste is the unfilled tail of a sequence's last block: fewer than 16 slots,
    and exactly ceil(L / 16) blocks per sequence, whatever the order of appends."""
    rng = np.random.default_rng(1)
    m = _bm(4000)
    for i in range(40):
        m.add(i, rng.integers(0, 50000, size=int(rng.integers(0, 300))).tolist())
    for _ in range(3000):
        m.append(int(rng.integers(0, 40)), int(rng.integers(0, 50000)))
    for i in range(40):
        L, nb = m.seq_len(i), len(m.seqs[i]["blocks"])
        assert nb == -(-L // 16) and nb * 16 - L < 16


def pin_bm_capacity_22048_tokens_640_per_request():
    """KV space of 22 048 tokens holds about 34 requests of 512 + 128 = 640 tokens (the
    serving-engine article, section 5): with 16-token blocks, 1378 blocks hold 34 whole
    requests and the 35th is refused."""
    import oracle.block_manager as obm
    m = _bm(22048 // 16, prefix=False)
    done = 0
    rng = np.random.default_rng(2)
    try:
        while True:
            m.add(done, rng.integers(0, 50000, size=512).tolist())
            for _ in range(128):
                m.append(done, int(rng.integers(0, 50000)))
            done += 1
    except obm.NoBlocks:
        pass
    assert done == 34 and 22048 // 640 == 34


def pin_bm_copy_on_write_parallel_sampling():
    """N samples share the prompt's blocks (count N); writing into the shared partial last
    block copies it first, so with 8 samples of a 3000-token prompt the first 7 appends copy
    and the last writes in place; full prompt blocks are never copied."""
    m = _bm(400)
    prompt = list(range(3000))
    m.add(0, prompt)
    for c in range(1, 8):
        m.fork(0, c)
    shared = list(m.seqs[0]["blocks"])
    assert len(shared) == 188 and all(m.ref[b] == 8 for b in shared)
    pairs = []
    for c in range(8):
        slot, src, dst = m.append(c, 5)
        if src >= 0:
            pairs.append((src, dst))
            assert slot == dst * 16 + 3000 % 16
        else:
            assert slot == shared[-1] * 16 + 3000 % 16
    assert len(pairs) == 7 and all(src == shared[-1] for src, _ in pairs)
    assert all(m.ref[b] == 8 for b in shared[:-1]) and m.ref[shared[-1]] == 1


def pin_bm_prefix_cache_3000_token_prefix():
    """A 3000-token shared prefix with 32-token private tails (serving-engine article,
    section 4): the second request finds the prefix's 187 full blocks (2992 tokens) in the
    cache, also after the first request has finished (its blocks stay cached)."""
    rng = np.random.default_rng(3)
    prefix = rng.integers(0, 50000, size=3000).tolist()
    m = _bm(1000)
    assert m.add(0, prefix + rng.integers(0, 50000, size=32).tolist()) == 0
    assert m.add(1, prefix + rng.integers(0, 50000, size=32).tolist()) == 187 * 16
    assert m.seqs[1]["blocks"][:187] == m.seqs[0]["blocks"][:187]
    m.free_seq(0)
    m.free_seq(1)
    assert m.add(2, prefix + [1] * 32) == 187 * 16


def pin_bm_key_chain_and_salt():
    """A key stands for the whole prefix: 16 equal tokens after a different first block give
    a different key (no hit), and the extra data (salt) separates otherwise equal prompts."""
    m = _bm(100)
    a = list(range(16)) + list(range(100, 116))
    b = list(range(1, 17)) + list(range(100, 116))
    m.add(0, a)
    assert m.add(1, b) == 0
    assert m.seqs[0]["keys"][1] != m.seqs[1]["keys"][1]
    assert m.add(2, a, salt=7) == 0
    assert m.add(3, a) == 32


def pin_bm_only_full_blocks_cached():
    m = _bm(100)
    m.add(0, list(range(20)))
    assert m.stats()[2] == 1
    assert m.add(1, list(range(20))) == 16


def pin_bm_evicts_least_recent_tail_first():
    """Released cached blocks keep their contents; under pressure the least recently used
    goes first, and a finished request's blocks enter the queue tail first, so its last
    block is evicted before its first."""
    m = _bm(4)
    m.add(0, list(range(48)))                       # blocks 0, 1, 2 (all full, cached)
    m.free_seq(0)
    assert m.evictable == [2, 1, 0] and m.free == [3]
    m.add(1, [9] * 16)                              # takes free block 3
    m.add(2, [8] * 16)                              # evicts block 2, the old tail
    assert m.seqs[2]["blocks"] == [2] and m.evictable == [1, 0]
    assert m.add(3, list(range(32))) == 32          # blocks 0, 1 still hit


def pin_bm_conservation_and_refcounts():
    """Every block is free, evictable or referenced, and a block's count is the number of
    tables holding it, through a random stream of adds, forks, appends and releases."""
    import oracle.block_manager as obm
    rng = np.random.default_rng(4)
    m = _bm(300)
    live, nxt = [], 0
    shared = rng.integers(0, 1000, size=64).tolist()
    for _ in range(2000):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                m.add(nxt, shared[:int(rng.integers(0, 64))] +
                      rng.integers(0, 1000, size=int(rng.integers(0, 40))).tolist())
                live.append(nxt)
                nxt += 1
            elif op == 1:
                m.fork(live[int(rng.integers(0, len(live)))], nxt)
                live.append(nxt)
                nxt += 1
            elif op == 2:
                m.append(live[int(rng.integers(0, len(live)))], int(rng.integers(0, 1000)))
            else:
                m.free_seq(live.pop(int(rng.integers(0, len(live)))))
        except obm.NoBlocks:
            pass
        count = [0] * m.N
        for s in m.seqs.values():
            for blk in s["blocks"]:
                count[blk] += 1
        assert count == m.ref
        used = sum(1 for c in count if c > 0)
        assert len(m.free) + len(m.evictable) + used == m.N
        assert not set(m.free) & set(m.evictable)


def pin_block_swap_round_trip():
    """Swapping blocks to a second pool and back restores them bit for bit; blocks not named
    stay as they were; pairs outside either pool are skipped."""
    rng = np.random.default_rng(5)
    dev = rng.integers(0, 1 << 16, size=(12, 16, 2, 8), dtype=np.uint16)
    host = np.zeros((6, 16, 2, 8), dtype=np.uint16)
    out_pairs = np.array([[3, 0], [7, 1], [11, 5], [12, 2], [2, 6]])   # last two skipped
    host2 = oracle.block_swap_ref(host, dev, out_pairs)
    assert np.array_equal(host2[[0, 1, 5]], dev[[3, 7, 11]])
    assert not host2[[2, 3, 4]].any()
    blank = np.zeros_like(dev)
    back = oracle.block_swap_ref(blank, host2, np.array([[0, 9], [1, 4], [5, 0]]))
    assert np.array_equal(back[[9, 4, 0]], dev[[3, 7, 11]])
    assert not np.delete(back, [9, 4, 0], axis=0).any()


def pin_bm_swap_preemption_keeps_contents():
    """Preemption by swapping: a victim's blocks go to host memory, its device blocks serve
    another sequence, and after swap-in every token of the victim reads the K/V it had
    (pools simulated with one label per slot, moved with the oracle's block swap)."""
    m = _bm(12, bs=4, prefix=False)
    m.set_host_blocks(10)
    dev = np.full((12, 4), -1, dtype=np.int64)
    host = np.full((10, 4), -1, dtype=np.int64)

    def write(seq, first, n, base):
        for i, slot in enumerate(m.slots(seq, first, n)):
            dev[slot // 4, slot % 4] = base + first + i

    m.add(7, list(range(12)))                      # device blocks 0-2, stays resident
    m.add(8, [1])                                  # device block 3, swapped out to host 0
    m.swap_out(8)
    m.add(0, list(range(17)))                      # device blocks 4-8
    write(0, 0, 17, 1000)
    before = [dev[sl // 4, sl % 4] for sl in m.slots(0, 0, 17)]
    pairs = m.swap_out(0)                          # to host blocks 1-5
    assert [tuple(p) for p in pairs] == [(4, 1), (5, 2), (6, 3), (7, 4), (8, 5)]
    host = oracle.block_swap_ref(host[:, :, None, None], dev[:, :, None, None],
                                 np.array(pairs))[:, :, 0, 0]
    assert m.stats()[0] == 9                       # its device blocks are free again
    m.add(1, list(range(100, 136)))                # a second sequence takes all 9 of them
    write(1, 0, 36, 5000)
    m.free_seq(1)
    back = m.swap_in(0)
    dev = oracle.block_swap_ref(dev[:, :, None, None], host[:, :, None, None],
                                np.array(back))[:, :, 0, 0]
    assert [dev[sl // 4, sl % 4] for sl in m.slots(0, 0, 17)] == before
    slot, _, _ = m.append(0, 3)
    assert slot // 4 == m.table(0, 5)[4]


# ----------------------------------------------------------------------------- per-head scales

def _fp8_case(seed=31, Hkv=4, G=2, d=64):
    w = wl.custom(batch=3, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=d,
                  kv_dtype="fp8_e4m3", context_lens=[5, 40, 77], seed=seed)
    return w


def pin_head_scales_equal_reduce_to_tensor():
    """One scale per kv head, all equal, is the per-tensor scale, bit for bit (decode and
    multi-token queries)."""
    w = _fp8_case()
    args = (w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    kw = dict(q_kind="bf16", kv_kind="fp8_e4m3")
    a = oracle.decode_ref(*args, k_scale=0.03, v_scale=0.5, **kw)
    b = oracle.decode_ref(*args, k_scale=[0.03] * 4, v_scale=[0.5] * 4, **kw)
    assert np.array_equal(a, b)
    qs = np.array([0, 1, 2, 3])
    a = oracle.prefill_ref(w.q, qs, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale,
                           k_scale=0.03, v_scale=0.5, **kw)
    b = oracle.prefill_ref(w.q, qs, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale,
                           k_scale=[0.03] * 4, v_scale=[0.5] * 4, **kw)
    assert np.array_equal(a, b)


def pin_head_scales_reach_their_own_heads():
    """kv head g uses scale[g]: with distinct per-head scales, the query heads of kv head g
    equal (bit for bit) a per-tensor run at scale[g]; the same for quantisation, head by
    head."""
    import oracle.quantize as qz
    w = _fp8_case(seed=32)
    ks, vs = [0.01, 0.02, 0.05, 0.11], [0.3, 0.7, 1.9, 0.05]
    kw = dict(q_kind="bf16", kv_kind="fp8_e4m3")
    args = (w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    per_head = oracle.decode_ref(*args, k_scale=ks, v_scale=vs, **kw)
    G = 2
    for g in range(4):
        one = oracle.decode_ref(*args, k_scale=ks[g], v_scale=vs[g], **kw)
        assert np.array_equal(per_head[:, g * G:(g + 1) * G], one[:, g * G:(g + 1) * G])
    rng = np.random.default_rng(33)
    new = rng.standard_normal((5, 4, 64)).astype(np.float32) * 3
    codes = qz.e4m3_encode(qz.quant_inputs(new, "f32", ks))
    for g in range(4):
        assert np.array_equal(codes[:, g], qz.e4m3_encode(qz.quant_inputs(new[:, g], "f32", ks[g])))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
