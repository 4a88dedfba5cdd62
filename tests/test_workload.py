"""Structure of the seeded synthetic inputs (CPU only)."""
import math

import numpy as np
import pytest

import workload as wl


def _check_tables(w):
    nb = (w.context_lens.astype(np.int64) + 15) // 16
    for b in range(w.batch):
        row = w.block_tables[b]
        assert (row[: nb[b]] >= 0).all() and (row[: nb[b]] < w.num_blocks).all()
        assert (row[nb[b]:] == -1).all()
        assert np.unique(row[: nb[b]]).size == nb[b]
        # the only waste is the last block's empty tail: fewer than 16 slots
        assert 0 <= nb[b] * 16 - w.context_lens[b] < 16 or w.context_lens[b] == 0


def test_deterministic():
    a, b = wl.make(1), wl.make(1)
    for f in ("q", "k_pool", "v_pool", "block_tables", "context_lens", "slot_mapping", "k_new"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c, d = wl.make(3, batch=8), wl.make(3, batch=8)
    assert np.array_equal(c.k_pool, d.k_pool) and np.array_equal(c.block_tables, d.block_tables)
    e = wl.make(3, batch=8, seed_offset=1)
    assert not np.array_equal(c.q, e.q)


def test_config1_shape_and_free_slots():
    w = wl.make(1)
    assert list(w.context_lens) == [1, 17, 100, 250]
    assert (w.num_blocks, w.num_q_heads, w.num_kv_heads, w.head_dim) == (64, 4, 4, 64)
    assert w.scale == 1 / 8
    _check_tables(w)
    used = wl.used_slot_mask(w).reshape(-1)
    assert w.block_tables[w.block_tables >= 0].size == 26
    assert np.unique(w.slot_mapping).size == 4 and not used[w.slot_mapping].any()


def test_config_lengths_full_size():
    L2 = wl.config_lengths(2)
    assert L2.size == 64 and L2.min() >= 128 and L2.max() <= 2048
    L3 = wl.config_lengths(3)
    assert L3.size == 256 and L3.min() >= 16 and L3.max() <= 8192
    assert 600 < np.median(L3) < 1600           # lognormal with median 1000
    L5 = wl.config_lengths(5)
    assert L5.size == 16 and L5.min() >= 16384 and L5.max() <= 32768


@pytest.mark.parametrize("idx,kw", [(2, dict(batch=6, len_range=(128, 700))),
                                    (3, dict(batch=12)),
                                    (5, dict(batch=2, len_range=(600, 1500)))])
def test_scattered_pools(idx, kw):
    w = wl.make(idx, **kw)
    _check_tables(w)
    nb = int(((w.context_lens + 15) // 16).sum())
    assert w.num_blocks == math.ceil(1.1 * nb)
    assert np.unique(w.block_tables[w.block_tables >= 0]).size == nb   # no sharing
    assert w.k_pool.shape == (w.num_blocks, 16, w.num_kv_heads, w.head_dim)


def test_config3_new_tokens_land_in_tail_slots():
    w = wl.make(3, batch=10)
    for b in range(w.batch):
        L = int(w.context_lens[b])
        s = int(w.slot_mapping[b])
        assert s // 16 == w.block_tables[b, (L - 1) // 16] and s % 16 == (L - 1) % 16


def test_config4_sharing_structure():
    w = wl.make(4)
    assert w.batch == 64 and (w.context_lens == 3032).all()
    assert w.copy_pairs.shape == (56, 2)               # 7 copies per prompt
    assert w.notes["unique_blocks"] == 1688
    assert w.slot_mapping.size == 64 * 32
    assert np.unique(w.slot_mapping).size == w.slot_mapping.size
    _check_tables(w)
    src, dst = w.copy_pairs[:, 0], w.copy_pairs[:, 1]
    assert np.unique(dst).size == dst.size and not np.isin(dst, src).any()


def test_fp8_quantisation_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32)
    s = float(np.abs(x).max()) / 448.0
    codes = wl.quantize_e4m3(x, s)
    import torch
    deq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
    y = np.abs(x.astype(np.float64) / s)
    normal = y >= 2.0 ** -6
    # round to nearest: half an ulp, i.e. 2^-4 relative for normals, 2^-10 absolute below
    assert (np.abs(deq - x)[normal] <= s * 2.0 ** -4 * y[normal] * (1 + 1e-12)).all()
    assert (np.abs(deq - x)[~normal] <= s * 2.0 ** -10 * (1 + 1e-12)).all()


def test_poison_marks_only_unused():
    w = wl.poison_unused(wl.make(3, batch=4))
    used = wl.used_slot_mask(w)
    assert (w.k_pool[~used] == wl.NAN_BITS["bf16"]).all()
    assert not (w.k_pool[used] == wl.NAN_BITS["bf16"]).all()


def test_kv_bytes_accounting():
    w = wl.make(1)
    assert w.kv_bytes == 368 * 2 * 4 * 64 * 4
