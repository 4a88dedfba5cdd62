"""Seeded synthetic inputs for paged decode attention.

This module builds inputs only: context lengths, block tables, physical pools filled
with random values, new tokens with their slots, and copy-on-write pairs. It holds
none of the attention arithmetic. Both the CPU oracle (in tests and the bench) and
the HIP path consume the arrays it returns.

Workloads (shapes from the pages' examples, sizes from the five named configurations):

  1  tiny fp32 MHA: B=4, context lens {1,17,100,250}, 4 heads, d=64, pool of 64
     blocks, tables sampled without replacement, 4 new tokens into free slots.
  2  Llama-2-7B-shaped fp16 MHA: B=64, L ~ U{128..2048}, 32 heads, d=128.
  3  Llama-3-8B-shaped bf16 GQA: B=256, L = clip(rint(LogNormal(ln 1000, 0.8)), 16, 8192),
     32 q heads over 8 kv heads, d=128, plus one new token per sequence in its tail slot.
  4  prefix sharing bf16 GQA: 8 prompts x 8 samples, 3000-token shared prefix,
     32-token private tail per sample, copy-on-write of the partial last shared block.
  5  long-context fp8-E4M3 KV: B=16, L ~ U{16384..32768}, GQA 32/8, d=128, per-tensor
     scales, 512-token split-KV partitions.

Multi-token queries (chunked prefill, prefix-cache tails): prefill_custom builds packed
query rows over a scattered pool for explicit query and context lengths;
chunked_prefill is the Llama-3-8B-shaped step of 16 prompts each prefilling its next
512-token chunk (a token budget of 8192; the LLM KV cache serving-engine article,
section 3, sweeps budgets of 512 to 8192), chunk index c ~ U{0..15}, so L = 512 (c + 1).

Block size is 16 everywhere (vLLM-PagedAttention与连续批处理技术拆解, section 3.1).
The pool layout is [num_blocks, block_size, kv_heads, head_dim] (AI vLLM: PagedAttention
不够用了之后, the paged_attention sketch's docstring); K and V are separate pools.

Storage encodings: f32 -> float32, f16 -> float16, bf16 -> uint16 bit patterns,
fp8_e4m3 -> uint8 bit patterns (OCP E4M3FN). Half and bfloat16 values are produced by
rounding float32 normals to nearest-even with torch on the CPU; fp8 values by scaling
with s = amax/448, clamping to +-448 and casting with torch's float8_e4m3fn.

Seeds: numpy PCG64 over SeedSequence(367 + config_index); child streams are spawned in
the fixed order lengths, placement, q, K, V, new tokens, slots.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16
SEED_BASE = 367

CONFIG_NAMES = {
    1: "tiny_fp32_mha",
    2: "llama2_7b_fp16_mha",
    3: "llama3_8b_gqa_bf16",
    4: "prefix_sharing_bf16_gqa",
    5: "long_context_fp8_gqa",
}

STORAGE_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3": np.uint8}
BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F}


@dataclass
class Workload:
    name: str
    index: int
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    kv_dtype: str
    q_dtype: str
    out_dtype: str
    scale: float
    k_scale: float
    v_scale: float
    partition_size: int
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, maxb], -1 padded
    q: np.ndarray                     # storage [B, Hq, d]
    k_pool: np.ndarray                # storage [N, bs, Hkv, d]
    v_pool: np.ndarray
    k_new: Optional[np.ndarray] = None    # storage [T, Hkv, d]
    v_new: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # int64 [T], -1 = skip
    copy_pairs: Optional[np.ndarray] = None    # int64 [P, 2] (src, dst)
    poisoned: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.batch else 0

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V one decode step must read: sum_b L_b * 2 * Hkv * d * bytes."""
        return self.total_tokens * 2 * self.num_kv_heads * self.head_dim * BYTES[self.kv_dtype]


# ----------------------------------------------------------------------------- helpers

def _to_storage(x: np.ndarray, kind: str) -> np.ndarray:
    """Round float32 values to the storage encoding (no scaling)."""
    if kind == "f32":
        return x.astype(np.float32, copy=False)
    if kind == "f16":
        return x.astype(np.float16)
    if kind == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(kind)


def quantize_e4m3(x: np.ndarray, s: float) -> np.ndarray:
    """clamp(x/s, +-448) cast to OCP E4M3FN with round-to-nearest-even; uint8 bits.

    Clamping comes first because torch casts out-of-range values to NaN."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = torch.clamp(t / np.float32(s), -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _normal_storage(rng: np.random.Generator, shape, kind: str, scale_out: Optional[list] = None):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if kind == "fp8_e4m3":
        amax = float(np.abs(x).max()) if x.size else 1.0
        s = amax / 448.0 if amax > 0 else 1.0
        if scale_out is not None:
            scale_out.append(s)
        return quantize_e4m3(x, s)
    return _to_storage(x, kind)


def _nblocks(L: np.ndarray, bs: int = BLOCK_SIZE) -> np.ndarray:
    return (L.astype(np.int64) + bs - 1) // bs


def _tables_from_ids(nb: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Assign ids (in (sequence, logical block) order) to rows; pad with -1."""
    maxb = max(1, int(nb.max()) if nb.size else 1)
    tab = np.full((nb.size, maxb), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nb):
        tab[b, :n] = ids[off:off + n]
        off += n
    return tab


def used_slot_mask(w: Workload) -> np.ndarray:
    """Boolean [N, bs]: True where a slot holds one of some sequence's first L tokens."""
    used = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        nb = (L + w.block_size - 1) // w.block_size
        for j in range(nb):
            n = min(w.block_size, L - j * w.block_size)
            used[w.block_tables[b, j], :n] = True
    return used


def poison_unused(w: Workload) -> Workload:
    """Fill every slot that holds no token of any sequence with NaN (in place)."""
    if w.kv_dtype == "f32":
        nan = np.float32(np.nan)
    elif w.kv_dtype == "f16":
        nan = np.uint16(NAN_BITS["f16"]).view(np.float16)
    else:
        nan = STORAGE_NP[w.kv_dtype](NAN_BITS[w.kv_dtype])
    free = ~used_slot_mask(w)
    w.k_pool[free] = nan
    w.v_pool[free] = nan
    w.poisoned = True
    return w


# ----------------------------------------------------------------------------- configs

def _children(index: int, seed_offset: int = 0):
    ss = np.random.SeedSequence(SEED_BASE + index + seed_offset)
    kids = ss.spawn(7)
    names = ["lengths", "placement", "q", "k", "v", "new", "slots"]
    return {n: np.random.Generator(np.random.PCG64(k)) for n, k in zip(names, kids)}


def _scattered_pool(nb: np.ndarray, rng: np.random.Generator, slack: float = 0.10):
    total = int(nb.sum())
    N = max(1, int(math.ceil((1.0 + slack) * total)))
    perm = rng.permutation(N)
    return N, _tables_from_ids(nb, perm[:total].astype(np.int32))


def _finish(name, index, seed, L, tables, N, Hq, Hkv, d, kv, qd, out, rngs,
            k_scale=None, v_scale=None, partition_size=0) -> Workload:
    B = L.size
    q = _normal_storage(rngs["q"], (B, Hq, d), qd)
    ks: list = []
    vs: list = []
    k_pool = _normal_storage(rngs["k"], (N, BLOCK_SIZE, Hkv, d), kv, ks)
    v_pool = _normal_storage(rngs["v"], (N, BLOCK_SIZE, Hkv, d), kv, vs)
    return Workload(
        name=name, index=index, seed=seed, batch=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=d, block_size=BLOCK_SIZE, num_blocks=N, kv_dtype=kv, q_dtype=qd,
        out_dtype=out, scale=1.0 / math.sqrt(d),
        k_scale=ks[0] if ks else 1.0, v_scale=vs[0] if vs else 1.0,
        partition_size=partition_size, context_lens=L.astype(np.int32), block_tables=tables,
        q=q, k_pool=k_pool, v_pool=v_pool)


def config_lengths(index: int, *, batch: Optional[int] = None,
                   len_range: Optional[tuple] = None, seed_offset: int = 0) -> np.ndarray:
    """Context lengths of configuration 2, 3 or 5 (first draw of the lengths stream)."""
    rng = _children(index, seed_offset)["lengths"]
    if index == 2:
        B = 64 if batch is None else batch
        lo, hi = (128, 2048) if len_range is None else len_range
        return rng.integers(lo, hi, size=B, endpoint=True)
    if index == 3:
        B = 256 if batch is None else batch
        x = rng.lognormal(mean=math.log(1000.0), sigma=0.8, size=B)
        L = np.clip(np.rint(x), 16, 8192).astype(np.int64)
        if len_range is not None:
            L = np.clip(L, len_range[0], len_range[1])
        return L
    if index == 5:
        B = 16 if batch is None else batch
        lo, hi = (16384, 32768) if len_range is None else len_range
        return rng.integers(lo, hi, size=B, endpoint=True)
    raise ValueError("configurations 1 and 4 have fixed lengths")


def make(index: int, *, batch: Optional[int] = None, len_range: Optional[tuple] = None,
         seed_offset: int = 0, poison: bool = False) -> Workload:
    """Build configuration `index` (1..5).

    batch / len_range shrink a configuration for parity runs the oracle finishes in
    seconds (same structure, fewer or shorter sequences); lengths drawn outside
    len_range are clipped into it. Configuration 4 takes batch as the prompt count.
    """
    if index not in CONFIG_NAMES:
        raise ValueError(f"unknown configuration {index}")
    seed = SEED_BASE + index + seed_offset
    rngs = _children(index, seed_offset)
    name = CONFIG_NAMES[index]

    if index == 1:
        L = np.array([1, 17, 100, 250], dtype=np.int64)
        if batch is not None:
            L = L[:batch]
        nb = _nblocks(L)
        N = 64
        ids = rngs["placement"].choice(N, size=int(nb.sum()), replace=False).astype(np.int32)
        tables = _tables_from_ids(nb, ids)
        w = _finish(name, index, seed, L, tables, N, 4, 4, 64, "f32", "f32", "f32", rngs)
        # four new tokens into distinct free slots (slots holding none of the first L tokens)
        free = np.flatnonzero(~used_slot_mask(w).reshape(-1))
        T = 4
        w.slot_mapping = rngs["slots"].choice(free, size=T, replace=False).astype(np.int64)
        w.k_new = _normal_storage(rngs["new"], (T, 4, 64), "f32")
        w.v_new = _normal_storage(rngs["new"], (T, 4, 64), "f32")

    elif index == 2:
        L = config_lengths(2, batch=batch, len_range=len_range, seed_offset=seed_offset)
        nb = _nblocks(L)
        N, tables = _scattered_pool(nb, rngs["placement"])
        w = _finish(name, index, seed, L, tables, N, 32, 32, 128, "f16", "f16", "f16", rngs)

    elif index == 3:
        L = config_lengths(3, batch=batch, len_range=len_range, seed_offset=seed_offset)
        B = L.size
        nb = _nblocks(L)
        N, tables = _scattered_pool(nb, rngs["placement"])
        w = _finish(name, index, seed, L, tables, N, 32, 8, 128, "bf16", "bf16", "bf16", rngs)
        # one new token per sequence; context_lens already count it, so it lands in
        # position L-1 of the sequence: slot = table[(L-1)//16]*16 + (L-1)%16
        pos = L - 1
        blk = tables[np.arange(B), pos // BLOCK_SIZE].astype(np.int64)
        w.slot_mapping = blk * BLOCK_SIZE + pos % BLOCK_SIZE
        w.k_new = _normal_storage(rngs["new"], (B, 8, 128), "bf16")
        w.v_new = _normal_storage(rngs["new"], (B, 8, 128), "bf16")

    elif index == 4:
        w = _make_prefix_sharing(rngs, seed, name, prompts=8 if batch is None else batch,
                                 samples=8, prefix=3000, tail=32)

    else:  # index == 5
        L = config_lengths(5, batch=batch, len_range=len_range, seed_offset=seed_offset)
        nb = _nblocks(L)
        N, tables = _scattered_pool(nb, rngs["placement"])
        w = _finish(name, index, seed, L, tables, N, 32, 8, 128, "fp8_e4m3", "bf16", "bf16",
                    rngs, partition_size=512)

    if poison:
        poison_unused(w)
    return w


def _make_prefix_sharing(rngs, seed, name, prompts, samples, prefix, tail) -> Workload:
    """Parallel sampling over shared prompts with copy-on-write of the partial block.

    Every sample's table references its prompt's full prefix blocks (refcount = samples).
    The last prefix block is partially filled; samples are visited in order and a
    sample whose next write would land in a block with refcount > 1 gets a private copy
    (a (src, dst) pair) and the refcount drops by one; the last sample writes the
    original in place. Tail tokens that do not fit go to freshly allocated blocks.
    """
    bs = BLOCK_SIZE
    Hq, Hkv, d = 32, 8, 128
    full = prefix // bs
    partial_fill = prefix % bs
    npre = full + (1 if partial_fill else 0)
    L_total = prefix + tail
    nb_seq = (L_total + bs - 1) // bs

    # logical allocation order -> physical ids through a seeded permutation
    per_prompt = npre + (samples - 1) * (1 if partial_fill else 0) + samples * (nb_seq - npre)
    total = prompts * per_prompt
    N = int(math.ceil(1.10 * total))
    perm = rngs["placement"].permutation(N).astype(np.int64)
    cursor = iter(perm[:total])

    B = prompts * samples
    tables = np.full((B, nb_seq), -1, dtype=np.int32)
    pairs = []
    refcount = {}
    for p in range(prompts):
        pre_ids = [int(next(cursor)) for _ in range(npre)]
        for i in pre_ids:
            refcount[i] = samples
        for s in range(samples):
            b = p * samples + s
            row = list(pre_ids)
            if partial_fill:
                last = row[-1]
                if refcount[last] > 1:
                    new = int(next(cursor))
                    pairs.append((last, new))
                    refcount[last] -= 1
                    refcount[new] = 1
                    row[-1] = new
            while len(row) < nb_seq:
                row.append(int(next(cursor)))
            tables[b] = row

    L = np.full(B, L_total, dtype=np.int64)
    w = _finish(name, 4, seed, L, tables, N, Hq, Hkv, d, "bf16", "bf16", "bf16", rngs)
    # tail tokens: positions prefix..prefix+tail-1 of every sample, written after the copies
    pos = np.arange(prefix, L_total, dtype=np.int64)
    slots = []
    for b in range(B):
        slots.append(tables[b, pos // bs].astype(np.int64) * bs + pos % bs)
    w.slot_mapping = np.concatenate(slots)
    T = w.slot_mapping.size
    w.k_new = _normal_storage(rngs["new"], (T, Hkv, d), "bf16")
    w.v_new = _normal_storage(rngs["new"], (T, Hkv, d), "bf16")
    w.copy_pairs = np.array(pairs, dtype=np.int64).reshape(-1, 2)
    w.notes = {"prompts": prompts, "samples": samples, "prefix": prefix, "tail": tail,
               "shared_full_blocks": full, "partial_fill": partial_fill,
               "unique_blocks": total}
    return w


def custom(*, batch, num_q_heads, num_kv_heads, head_dim, kv_dtype, q_dtype=None,
           out_dtype=None, context_lens, seed=0, num_blocks=None, slack=0.10,
           partition_size=0) -> Workload:
    """A scattered-pool workload with explicit shape and lengths (edge-case tests)."""
    rngs = _children(100, seed)
    L = np.asarray(context_lens, dtype=np.int64).reshape(batch)
    nb = _nblocks(L)
    total = int(nb.sum())
    N = max(1, int(math.ceil((1.0 + slack) * total))) if num_blocks is None else num_blocks
    if N < total:
        raise ValueError("pool too small")
    perm = rngs["placement"].permutation(N).astype(np.int32)
    tables = _tables_from_ids(nb, perm[:total])
    qd = q_dtype or ("bf16" if kv_dtype == "fp8_e4m3" else kv_dtype)
    od = out_dtype or qd
    return _finish(f"custom_g{num_q_heads // num_kv_heads}_d{head_dim}_{kv_dtype}", 0,
                   SEED_BASE + 100 + seed, L, tables, N, num_q_heads, num_kv_heads, head_dim,
                   kv_dtype, qd, od, rngs, partition_size=partition_size)


# ----------------------------------------------------------------------------- multi-token queries

@dataclass
class PrefillWorkload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    kv_dtype: str
    q_dtype: str
    out_dtype: str
    scale: float
    k_scale: float
    v_scale: float
    context_lens: np.ndarray          # int32 [B]
    query_start: np.ndarray           # int32 [B + 1]
    block_tables: np.ndarray          # int32 [B, maxb], -1 padded
    q: np.ndarray                     # storage [Tq, Hq, d]
    k_pool: np.ndarray                # storage [N, bs, Hkv, d]
    v_pool: np.ndarray

    @property
    def batch(self) -> int:
        return int(self.context_lens.size)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start.astype(np.int64))

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.batch else 0

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start[-1])


def prefill_custom(*, query_lens, context_lens, num_q_heads, num_kv_heads, head_dim,
                   kv_dtype, q_dtype=None, out_dtype=None, seed=0, slack=0.10,
                   name=None) -> PrefillWorkload:
    """Packed query rows (query_lens[b] for sequence b) over a scattered pool holding
    context_lens[b] tokens per sequence; the query tokens are the last ones of each."""
    rngs = _children(200, seed)
    L = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    n = np.asarray(query_lens, dtype=np.int64).reshape(-1)
    if n.shape != L.shape:
        raise ValueError("one query length per sequence")
    nb = _nblocks(L)
    N, tables = _scattered_pool(nb, rngs["placement"], slack)
    qd = q_dtype or ("bf16" if kv_dtype == "fp8_e4m3" else kv_dtype)
    od = out_dtype or qd
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = _normal_storage(rngs["q"], (int(qs[-1]), num_q_heads, head_dim), qd)
    ks: list = []
    vs: list = []
    k_pool = _normal_storage(rngs["k"], (N, BLOCK_SIZE, num_kv_heads, head_dim), kv_dtype, ks)
    v_pool = _normal_storage(rngs["v"], (N, BLOCK_SIZE, num_kv_heads, head_dim), kv_dtype, vs)
    return PrefillWorkload(
        name=name or f"prefill_g{num_q_heads // num_kv_heads}_d{head_dim}_{kv_dtype}",
        seed=SEED_BASE + 200 + seed, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, num_blocks=N, kv_dtype=kv_dtype, q_dtype=qd, out_dtype=od,
        scale=1.0 / math.sqrt(head_dim), k_scale=ks[0] if ks else 1.0,
        v_scale=vs[0] if vs else 1.0, context_lens=L.astype(np.int32), query_start=qs,
        block_tables=tables, q=q, k_pool=k_pool, v_pool=v_pool)


def chunked_prefill(*, batch: int = 16, chunk: int = 512, max_chunks: int = 16,
                    seed_offset: int = 0) -> PrefillWorkload:
    """One chunked-prefill step of a Llama-3-8B-shaped layer (32 q heads over 8 kv heads,
    d=128, bf16): `batch` prompts, each with c ~ U{0..max_chunks-1} chunks already cached
    and its next `chunk` tokens as queries, so L = chunk * (c + 1) and n = chunk."""
    rng = _children(201, seed_offset)["lengths"]
    c = rng.integers(0, max_chunks, size=batch)
    L = chunk * (c + 1)
    return prefill_custom(query_lens=np.full(batch, chunk), context_lens=L, num_q_heads=32,
                          num_kv_heads=8, head_dim=128, kv_dtype="bf16", seed=1 + seed_offset,
                          name="chunked_prefill_llama3_8b_bf16")
