"""Parity of the default split's cut-segment merge at engineered chunk boundaries.

With 8 kv heads per workgroup the decode deals T units (16-token blocks of a sequence,
per head group) into W = 256 static chunks [T*r/W, T*(r+1)/W). Choosing the block counts
makes the chunk boundaries fall exactly where the merge's cases differ: a segment that
begins exactly at a chunk boundary and ends in the next chunk, segments that are exactly
one or two chunks, segments over many chunks with empty chunks among them (T < W), zero
lengths in between, and two head groups per sequence. Every case runs with bf16 and with
fp8 K/V (d = 128); every output is compared with the oracle (max-abs error 1e-2 for bf16,
5e-2 for fp8).
"""
import numpy as np
import pytest

import workload as wl
from tests.gpu_harness import TOL, as_f64, gpu_decode, max_abs_err, oracle_decode, to_device

pytestmark = pytest.mark.gpu

W = 256   # static chunks for 8 kv heads per workgroup (8 waves per CU on 256 CUs)

# (K/V type, tokens per decode unit) at d = 128
KINDS = [("bf16", 16), ("fp8_e4m3", 16)]


@pytest.fixture(params=KINDS, ids=[k for k, _ in KINDS])
def kind(request):
    return request.param


def _lengths(units, seed, ut):
    """Context lengths with exactly the given unit counts (units of ut tokens), ragged
    inside the last unit."""
    rng = np.random.default_rng(seed)
    nu = np.asarray(units, dtype=np.int64)
    tail = rng.integers(1, ut + 1, size=nu.size)
    return np.where(nu > 0, (nu - 1) * ut + tail, 0)


def _run(units, kind, num_kv_heads=8, num_q_heads=32, seed=0):
    """Decode the workload twice: with its own table width, and with the tables padded
    (-1) so wide that a call could have 8 units per chunk. With at least W/4 segments the
    wide run selects the per-chunk merge; fewer segments, or fewer possible units, select
    the per-(kv head, sequence) merge."""
    import torch
    kv, ut = kind
    L = _lengths(units, seed, ut)
    w = wl.custom(batch=L.size, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  head_dim=128, kv_dtype=kv, context_lens=L, seed=seed)
    ref = oracle_decode(w)
    d = to_device(w)
    groups = num_kv_heads // 8
    wide_units = -(-8 * W // (groups * L.size))
    width = max(w.block_tables.shape[1], wide_units * (ut // 16))
    wide = np.full((L.size, width), -1, dtype=np.int32)
    wide[:, :w.block_tables.shape[1]] = w.block_tables
    for tables, max_len in ((d["tables"], w.max_context_len),
                            (torch.from_numpy(wide).cuda(), 16 * width)):
        dd = dict(d, tables=tables)
        out = as_f64(gpu_decode(w, dd, max_context_len=max_len))
        err = max_abs_err(out, ref)
        assert err <= TOL[kv], (max_len, err)
    return w


def test_segment_starting_at_a_chunk_boundary_ends_in_the_next(kind):
    # units 6, 2, 6, 2, ...: T = 1024, chunks of 4 units; each 6-unit sequence starts a
    # chunk and ends two units into the next one
    units = [6, 2] * 128
    assert sum(units) == 4 * W
    _run(units, kind)


def test_segments_of_exactly_one_and_two_chunks(kind):
    _run([4] * 256, kind)                # every sequence is one whole chunk: nothing cut
    _run([8] * 128, kind, seed=1)        # every sequence is exactly two chunks


@pytest.mark.parametrize("pad", [0, 56])
def test_segments_over_many_chunks_with_empty_chunks_and_zero_lengths(kind, pad):
    # T = 255 < W: one static chunk is empty; the 100-unit sequence spans 100 chunks.
    # With 56 more empty sequences there are W/4 segments, so the wide run takes the
    # per-chunk merge over the same chunks.
    units = [100, 0, 50, 60, 0, 30, 10, 5] + [0] * pad
    assert sum(units) == W - 1
    _run(units, kind, seed=2)


def test_long_segments_spanning_several_chunks(kind):
    # T = 2048 (chunks of 8 units); sequences of 3..40 units cut once or many times
    rng = np.random.default_rng(3)
    units = list(rng.integers(3, 41, size=90))
    units.append(2048 - sum(units))
    assert units[-1] > 0
    _run(units, kind, seed=3)


def test_two_head_groups_per_sequence(kind):
    # 16 kv heads: two head groups, so a sequence is two segments of nb units each
    units = [6, 2] * 64
    assert 2 * sum(units) == 4 * W
    _run(units, kind, num_kv_heads=16, num_q_heads=32, seed=4)


@pytest.mark.parametrize("L", [4096, 8191, 300])
@pytest.mark.parametrize("pad", [0, 63])
def test_single_long_sequence(kind, L, pad):
    # one non-empty sequence: its blocks are spread over every chunk (one unit per chunk
    # for 4096 tokens), so its merge folds up to 256 pieces; with 63 empty sequences
    # beside it the wide run folds them in the per-chunk merge
    _run([-(-L // kind[1])] + [0] * pad, kind, seed=5)
