"""Per-kv-head fp8 scales on the GPU (pa_cache_write_fp8_head_scales, pa_decode_head_scales,
pa_prefill_head_scales) against the oracle: quantisation bytes bit-exact; attention within
the fp8 tolerance (oracle on the dequantised values, each kv head times its own scale); all
scales equal gives bitwise the per-tensor calls."""
import numpy as np
import pytest

import oracle
import workload as wl
import paged_kv_cache_367_amd as pa
from gpu_harness import TOL, as_f64, max_abs_err, torch_from_storage
from test_gpu_cache_ops import _quant_case

pytestmark = pytest.mark.gpu

# amax / 448 for per-head value ranges of 1 to 8, as a per-head calibration would give:
# dequantised K/V stay O(1), so the bf16 output rounding stays far below the tolerance
K_SCALES = [c / 448.0 for c in (3.0, 5.5, 2.0, 8.0, 4.2, 1.1, 6.6, 3.9)]
V_SCALES = [c / 448.0 for c in (4.0, 2.2, 5.0, 1.5, 7.0, 3.3, 2.8, 6.1)]


def _t(x):
    import torch
    return torch.tensor(x, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16"])
def test_cache_write_fp8_head_scales_bit_exact(kind):
    import torch
    rng = np.random.default_rng(41)
    N, Hkv, d, T = 40, 8, 128, 150
    k_pool = rng.integers(0, 256, size=(N, 16, Hkv, d), dtype=np.uint8)
    v_pool = rng.integers(0, 256, size=(N, 16, Hkv, d), dtype=np.uint8)
    slots = rng.choice(N * 16, size=T, replace=False).astype(np.int64)
    slots[5] = -1
    # rows spanning each head's range, with code midpoints, saturation, inf and NaN at the
    # first head's scale (the same data is also far out of range for the smaller scales)
    k_store, k_dev = _quant_case(kind, T, Hkv, d, K_SCALES[0], 3)
    v_store, v_dev = _quant_case(kind, T, Hkv, d, V_SCALES[0], 4)
    kp, vp = torch.from_numpy(k_pool).cuda(), torch.from_numpy(v_pool).cuda()
    pa.pa_cache_write_fp8(kp, vp, k_dev, v_dev, torch.from_numpy(slots).cuda(),
                          k_scale=_t(K_SCALES), v_scale=_t(V_SCALES))
    torch.cuda.synchronize()
    assert np.array_equal(kp.cpu().numpy(),
                          oracle.cache_write_fp8_ref(k_pool, k_store, kind, K_SCALES, slots))
    assert np.array_equal(vp.cpu().numpy(),
                          oracle.cache_write_fp8_ref(v_pool, v_store, kind, V_SCALES, slots))


def _fp8_workload(seed):
    return wl.custom(batch=6, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_dtype="fp8_e4m3",
                     context_lens=[1, 16, 17, 300, 1000, 2200], seed=seed)


def test_decode_head_scales_against_oracle():
    import torch
    w = _fp8_workload(43)
    q, k, v = (torch_from_storage(a, kind) for a, kind in
               ((w.q, "bf16"), (w.k_pool, "fp8_e4m3"), (w.v_pool, "fp8_e4m3")))
    tab, lens = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda()
    for part in (0, 256):
        out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
        pa.pa_decode(out, q, k, v, tab, lens, w.max_context_len, w.scale, k_scale=_t(K_SCALES),
                     v_scale=_t(V_SCALES), partition_size=part)
        torch.cuda.synchronize()
        want = oracle.decode_ref(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens,
                                 w.scale, q_kind="bf16", kv_kind="fp8_e4m3", k_scale=K_SCALES,
                                 v_scale=V_SCALES)
        err = max_abs_err(as_f64(out), want)
        print(f"decode per-head scales, partition {part}: max_abs_err={err:.3e}")
        assert err <= TOL["fp8_e4m3"]


def test_prefill_head_scales_against_oracle():
    import torch
    w = wl.prefill_custom(query_lens=[1, 30, 70], context_lens=[10, 30, 400], num_q_heads=32,
                          num_kv_heads=8, head_dim=128, kv_dtype="fp8_e4m3", seed=45)
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    pa.pa_prefill(out, torch_from_storage(w.q, "bf16"), torch_from_storage(w.k_pool, "fp8_e4m3"),
                  torch_from_storage(w.v_pool, "fp8_e4m3"), torch.from_numpy(w.block_tables).cuda(),
                  torch.from_numpy(w.context_lens).cuda(), torch.from_numpy(w.query_start).cuda(),
                  w.max_query_len, w.scale, k_scale=_t(K_SCALES), v_scale=_t(V_SCALES))
    torch.cuda.synchronize()
    want = oracle.prefill_ref(w.q, w.query_start, w.k_pool, w.v_pool, w.block_tables,
                              w.context_lens, w.scale, q_kind="bf16", kv_kind="fp8_e4m3",
                              k_scale=K_SCALES, v_scale=V_SCALES)
    assert max_abs_err(as_f64(out), want) <= TOL["fp8_e4m3"]


def test_equal_head_scales_are_the_per_tensor_calls():
    import torch
    w = _fp8_workload(47)
    q, k, v = (torch_from_storage(a, kind) for a, kind in
               ((w.q, "bf16"), (w.k_pool, "fp8_e4m3"), (w.v_pool, "fp8_e4m3")))
    tab, lens = torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda()
    a = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    pa.pa_decode(a, q, k, v, tab, lens, w.max_context_len, w.scale, k_scale=0.03, v_scale=0.7)
    pa.pa_decode(b, q, k, v, tab, lens, w.max_context_len, w.scale, k_scale=_t([0.03] * 8),
                 v_scale=_t([0.7] * 8))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the slot write: one scale for all heads either way
    rng = np.random.default_rng(49)
    T = 40
    new = torch.from_numpy(rng.standard_normal((T, 8, 128)).astype(np.float32)).cuda()
    slots = torch.from_numpy(rng.choice(w.num_blocks * 16, size=T, replace=False)).cuda()
    k1, v1 = k.clone(), v.clone()
    k2, v2 = k.clone(), v.clone()
    pa.pa_cache_write_fp8(k1, v1, new, new, slots, k_scale=0.0123, v_scale=0.5)
    pa.pa_cache_write_fp8(k2, v2, new, new, slots, k_scale=_t([0.0123] * 8),
                          v_scale=_t([0.5] * 8))
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)


def test_quantise_per_head_then_decode():
    """New tokens quantised with per-head scales, then decode with the same scales: within
    the fp8 tolerance of the oracle run on the written (dequantised) pools."""
    import torch
    w = _fp8_workload(51)
    rng = np.random.default_rng(53)
    B = w.batch
    L = w.context_lens.astype(np.int64)
    pos = L - 1                                    # each sequence's newest token
    slots = (w.block_tables[np.arange(B), pos // 16].astype(np.int64) * 16 + pos % 16)
    new_k = (rng.standard_normal((B, 8, 128)) * np.array(K_SCALES)[None, :, None] * 120)
    new_v = (rng.standard_normal((B, 8, 128)) * np.array(V_SCALES)[None, :, None] * 120)
    nk, nv = new_k.astype(np.float32), new_v.astype(np.float32)
    k, v = torch_from_storage(w.k_pool, "fp8_e4m3"), torch_from_storage(w.v_pool, "fp8_e4m3")
    pa.pa_cache_write_fp8(k, v, torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda(),
                          torch.from_numpy(slots).cuda(), k_scale=_t(K_SCALES),
                          v_scale=_t(V_SCALES))
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device="cuda")
    pa.pa_decode(out, torch_from_storage(w.q, "bf16"), k, v,
                 torch.from_numpy(w.block_tables).cuda(), torch.from_numpy(w.context_lens).cuda(),
                 w.max_context_len, w.scale, k_scale=_t(K_SCALES), v_scale=_t(V_SCALES))
    torch.cuda.synchronize()
    k_ref = oracle.cache_write_fp8_ref(w.k_pool, nk, "f32", K_SCALES, slots)
    v_ref = oracle.cache_write_fp8_ref(w.v_pool, nv, "f32", V_SCALES, slots)
    assert np.array_equal(k.cpu().numpy(), k_ref) and np.array_equal(v.cpu().numpy(), v_ref)
    want = oracle.decode_ref(w.q, k_ref, v_ref, w.block_tables, w.context_lens, w.scale,
                             q_kind="bf16", kv_kind="fp8_e4m3", k_scale=K_SCALES,
                             v_scale=V_SCALES)
    assert max_abs_err(as_f64(out), want) <= TOL["fp8_e4m3"]
