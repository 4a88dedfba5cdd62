"""Decode attention on the GPU against the fp64 oracle on the same seeded inputs.

Sizes here are ones the oracle finishes in seconds but still span several blocks,
partitions and waves with a ragged tail. Tolerances are max-abs error: 1e-5 for fp32
KV, 1e-2 for fp16/bf16 KV, 5e-2 for fp8-E4M3 KV (oracle on the dequantised values).
"""
import numpy as np
import pytest

import workload as wl
from gpu_harness import (TOL, as_f64, gpu_decode, gpu_step, max_abs_err, oracle_decode,
                         oracle_pools_after_step, to_device)

pytestmark = pytest.mark.gpu


def _check(w, out, ref, tol=None):
    err = max_abs_err(as_f64(out), ref)
    print(f"{w.name}: B={w.batch} G={w.group} d={w.head_dim} kv={w.kv_dtype} "
          f"max_abs_err={err:.3e}", flush=True)
    assert err <= (TOL[w.kv_dtype] if tol is None else tol)
    return err


def test_config1_tiny_fp32():
    w = wl.make(1)
    d = to_device(w)
    before = gpu_decode(w, d)
    _check(w, before, oracle_decode(w))
    out = gpu_step(w, d)                       # writes go to free slots: decode unchanged
    assert np.array_equal(as_f64(out), as_f64(before))


@pytest.mark.parametrize("idx,kw", [
    (2, dict(batch=6, len_range=(128, 700))),
    (3, dict(batch=24)),
    (4, dict(batch=1)),
    (5, dict(batch=2, len_range=(1500, 2600))),
])
def test_configs_reduced(idx, kw):
    w = wl.make(idx, **kw)
    d = to_device(w)
    out = gpu_step(w, d, partition_size=w.partition_size)
    k, v = oracle_pools_after_step(w)
    _check(w, out, oracle_decode(w, k, v))


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16", "fp8_e4m3"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_group_dim_dtype_grid(kv, G, d):
    lens = [1, 15, 16, 17, 33, 160, 511, 512, 513, 1100]
    w = wl.custom(batch=len(lens), num_q_heads=2 * G, num_kv_heads=2, head_dim=d,
                  kv_dtype=kv, context_lens=lens, seed=G * 1000 + d)
    if kv == "fp8_e4m3":
        w.k_scale, w.v_scale = 0.02, 0.03
    dev = to_device(w)
    _check(w, gpu_decode(w, dev, partition_size=256), oracle_decode(w))


@pytest.mark.parametrize("part", [0, 16, 64, 256, 512, 1024, 4096])
def test_partition_sizes(part):
    w = wl.make(3, batch=12, len_range=(16, 3000))
    d = to_device(w)
    _check(w, gpu_decode(w, d, partition_size=part), oracle_decode(w))


# With an fp32 output only the kernel's arithmetic is left. The matrix cores take every
# softmax weight p as a hi and a lo 16-bit part (hi + lo within 2^-16 of p for bf16 and
# fp8 K/V, 2^-22 for fp16) and the normaliser sums p itself, so the output is off by at
# most about 2^-16 of the spread |v - out| plus fp32 rounding: a few 1e-5 here.
FP32_OUT_TOL = {"f16": 2e-3, "bf16": 2e-3, "fp8_e4m3": 2e-3}


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8_e4m3"])
def test_fp32_output_tightens_error(kv):
    """With an fp32 output the only error left is the kernel's own arithmetic."""
    w = wl.custom(batch=5, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype=kv,
                  context_lens=[3, 64, 400, 777, 1500], seed=7)
    dev = to_device(w)
    out = gpu_decode(w, dev, out_dtype="f32")
    _check(w, out, oracle_decode(w), tol=FP32_OUT_TOL[kv])


def test_nan_in_unused_slots_changes_nothing():
    clean = wl.make(3, batch=16)
    dirty = wl.make(3, batch=16, poison=True)
    a = gpu_decode(clean, to_device(clean), partition_size=256)
    b = gpu_decode(dirty, to_device(dirty), partition_size=256)
    assert np.isfinite(as_f64(b)).all()
    assert np.array_equal(as_f64(a), as_f64(b))
    _check(dirty, b, oracle_decode(dirty))


def test_block_placement_is_bitwise_irrelevant():
    w = wl.make(3, batch=16)
    a = gpu_decode(w, to_device(w), partition_size=256)
    perm = np.random.default_rng(11).permutation(w.num_blocks)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    w.k_pool, w.v_pool = k2, v2
    w.block_tables = np.where(w.block_tables >= 0, perm[np.maximum(w.block_tables, 0)],
                              -1).astype(np.int32)
    b = gpu_decode(w, to_device(w), partition_size=256)
    assert np.array_equal(as_f64(a), as_f64(b))


def test_zero_and_single_token_lengths():
    w = wl.custom(batch=6, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="bf16",
                  context_lens=[0, 1, 0, 16, 1, 600], seed=3)
    out = as_f64(gpu_decode(w, to_device(w), partition_size=512))
    ref = oracle_decode(w)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.array_equal(out[1], ref[1]) and np.array_equal(out[4], ref[4])   # exact V row
    assert max_abs_err(out, ref) <= TOL["bf16"]


def test_all_lengths_zero():
    w = wl.custom(batch=3, num_q_heads=8, num_kv_heads=2, head_dim=64, kv_dtype="f16",
                  context_lens=[0, 0, 0], seed=1, num_blocks=4)
    assert (as_f64(gpu_decode(w, to_device(w))) == 0).all()


def test_full_table_width_and_max_context():
    """L equal to the table width (every entry used) and max_context_len at its cap."""
    lens = [32 * 16, 32 * 16 - 5, 7]
    w = wl.custom(batch=3, num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype="bf16",
                  context_lens=lens, seed=9)
    assert w.block_tables.shape[1] == 32
    _check(w, gpu_decode(w, to_device(w), partition_size=128, max_context_len=32 * 16),
           oracle_decode(w))


def test_shared_blocks_across_sequences():
    """Configuration 4's structure: 8 samples read the same prefix blocks."""
    w = wl.make(4, batch=1)
    d = to_device(w)
    out = gpu_step(w, d)
    k, v = oracle_pools_after_step(w)
    _check(w, out, oracle_decode(w, k, v))


def test_error_codes_on_device_buffers():
    import torch
    import paged_kv_cache_367_amd as pa
    w = wl.make(3, batch=4, len_range=(600, 2000))
    d = to_device(w)
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode(out, d["q"], d["k"], d["v"], d["tables"], d["lens"], w.max_context_len,
                     w.scale, workspace=small, partition_size=512)
    assert e.value.status == -5


@pytest.mark.parametrize("part", [0, 16, 64])
@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_out_of_pool_block_ids_are_masked(kv, part):
    """A table entry below L that lies outside [0, num_blocks) is never dereferenced and
    its 16 tokens are left out of the softmax: the result equals the attention over the
    sequence's other tokens (attention does not depend on token order), and a sequence
    whose blocks are all outside the pool gives zeros; bf16 and fp8 K/V, the default split
    and two partition sizes."""
    import dataclasses
    lens = [100, 40, 64, 17]
    w = wl.custom(batch=4, num_q_heads=16, num_kv_heads=4, head_dim=128, kv_dtype=kv,
                  context_lens=lens, seed=21)
    N = w.num_blocks
    bad = w.block_tables.copy()
    bad[0, 2] = N + 5          # a full block in the middle
    bad[1, 0] = -7             # the first block
    bad[2, 3] = N + 1          # the last block
    bad[3, :2] = [N, 2 ** 31 - 1]   # every block of the sequence
    # the same attention written with valid tables: the bad blocks' tokens removed
    good = np.full_like(bad, -1)
    good[0, :6] = np.delete(w.block_tables[0, :7], 2)
    good[1, :2] = w.block_tables[1, 1:3]
    good[2, :3] = w.block_tables[2, :3]
    exp = dataclasses.replace(w, block_tables=good,
                              context_lens=np.array([84, 24, 48, 0], dtype=np.int32))
    ref = oracle_decode(exp)
    w_bad = dataclasses.replace(w, block_tables=bad)
    out = as_f64(gpu_decode(w_bad, to_device(w_bad), partition_size=part, out_dtype="f32"))
    assert (out[3] == 0).all()
    err = max_abs_err(out, ref)
    print(f"out-of-pool ids, {kv}, partition {part}: max_abs_err={err:.3e}", flush=True)
    assert err <= FP32_OUT_TOL[kv]


@pytest.mark.parametrize("part", [0, 256])
def test_workspace_contents_do_not_matter(part):
    """The workspace needs no initialisation: one filled with 0xFF bytes (NaN floats,
    negative headers) and one filled with zeros give the same bits, call after call."""
    import torch
    import paged_kv_cache_367_amd as pa
    w = wl.make(3, batch=40, len_range=(16, 2500))
    d = to_device(w)
    outs = []
    for fill in (0x00, 0xFF, 0xFF):
        desc = pa.binding.make_desc(d["q"], d["k"], d["tables"], None, part)
        ws = pa.binding.decode_workspace(desc, w.max_context_len)
        ws.fill_(fill)
        out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
        pa.pa_decode(out, d["q"], d["k"], d["v"], d["tables"], d["lens"], w.max_context_len,
                     w.scale, workspace=ws, partition_size=part)
        torch.cuda.synchronize()
        outs.append(as_f64(out))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    _check(w, torch.from_numpy(outs[0]), oracle_decode(w))


@pytest.mark.parametrize("kv", ["f32", "bf16", "f16", "fp8_e4m3"])
@pytest.mark.parametrize("scale", [-0.09, 0.0, 1.7])
def test_negative_zero_and_large_score_scales(kv, scale):
    """The matrix-core path folds the score scale into the exponent and moves a negative
    scale onto q as a sign flip; a zero scale gives equal weights (the mean of the V rows
    below L). fp8 also takes a negative k_scale, which enters the score scale. (Not fp32 at
    19 times 1/sqrt(d): logits of several tens carry fp32 rounding of about 1e-5 of their
    size into the weights, the size of the fp32 bar itself.)"""
    import dataclasses
    if kv == "f32" and abs(scale) > 1.0:
        pytest.skip("fp32 bar of 1e-5 is for scales near 1/sqrt(d)")
    lens = [1, 16, 17, 100, 700]
    w = wl.custom(batch=len(lens), num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype=kv,
                  context_lens=lens, seed=31)
    w = dataclasses.replace(w, scale=scale)
    if kv == "fp8_e4m3":
        w = dataclasses.replace(w, k_scale=-w.k_scale)
    dev = to_device(w)
    for part in (0, 64):
        _check(w, gpu_decode(w, dev, partition_size=part), oracle_decode(w))


@pytest.mark.parametrize("kv,part", [("bf16", 0), ("fp8_e4m3", 0), ("fp8_e4m3", 64)])
def test_largest_batch(kv, part):
    """4096 sequences, the most a call takes (their lengths and prefix sums fill LDS), with
    lengths 0..40 (empty, one-block and two-block sequences side by side); every output
    against the oracle."""
    rng = np.random.default_rng(77)
    lens = rng.integers(0, 41, size=4096)
    w = wl.custom(batch=4096, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype=kv,
                  context_lens=lens, seed=77)
    _check(w, gpu_decode(w, to_device(w), partition_size=part), oracle_decode(w))
