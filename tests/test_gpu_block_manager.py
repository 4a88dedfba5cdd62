"""The block manager driving the kernels: prompts that share a prefix (the second hits the
prefix cache), forked samples whose appends copy the shared partial block on write, then
decode over the manager's tables. The native manager's tables, slots and copy pairs run the
HIP slot write, block copy and decode; the oracle's manager, fed the same operations, builds
the host pools with the oracle's slot write and block copy. Pools must be equal bit for bit
and the decode within the bf16 tolerance."""
import numpy as np
import pytest

import oracle
import oracle.block_manager as obm
import paged_kv_cache_367_amd as pa
from gpu_harness import TOL, as_f64, max_abs_err, torch_from_storage

pytestmark = pytest.mark.gpu

HKV, G, D, BS, N = 2, 4, 128, 16, 96


def _bf16(rng, shape):
    import torch
    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def test_manager_drives_write_copy_decode():
    import torch
    rng = np.random.default_rng(11)
    nat, ref = pa.BlockManager(N, BS), obm.BlockManager(N, BS)
    k_host = _bf16(rng, (N, BS, HKV, D))
    v_host = _bf16(rng, (N, BS, HKV, D))
    k_dev, v_dev = torch_from_storage(k_host, "bf16"), torch_from_storage(v_host, "bf16")

    def write(slots, k_rows, v_rows):
        nonlocal k_host, v_host
        s = np.asarray(slots, dtype=np.int64)
        pa.pa_cache_write(k_dev, v_dev, torch_from_storage(k_rows, "bf16"),
                          torch_from_storage(v_rows, "bf16"), torch.from_numpy(s).cuda())
        k_host = oracle.cache_write_ref(k_host, k_rows, s)
        v_host = oracle.cache_write_ref(v_host, v_rows, s)

    def copy(src, dst):
        nonlocal k_host, v_host
        pairs = np.array([[src, dst]], dtype=np.int64)
        pa.pa_block_copy(k_dev, v_dev, torch.from_numpy(pairs).cuda())
        k_host = oracle.block_copy_ref(k_host, pairs)
        v_host = oracle.block_copy_ref(v_host, pairs)

    prefix = rng.integers(0, 30000, size=200).tolist()
    p0 = prefix + rng.integers(0, 30000, size=27).tolist()
    p1 = prefix + rng.integers(0, 30000, size=9).tolist()
    # sequence 1 finds the 12 full prefix blocks; sequence 7 (the same prompt as 1) also
    # finds sequence 1's 13th block, full since its prefill
    for sid, toks, want_cached in [(0, p0, 0), (1, p1, 192), (7, p1, 208)]:
        cached = nat.add(sid, toks)
        assert cached == ref.add(sid, toks) == want_cached
        n = len(toks) - cached
        slots = nat.slots(sid, cached, n)
        assert slots.tolist() == ref.slots(sid, cached, n)
        write(slots, _bf16(rng, (n, HKV, D)), _bf16(rng, (n, HKV, D)))

    for c in (2, 3, 4):
        nat.fork(0, c)
        ref.fork(0, c)
    copies = 0
    for step in range(5):
        for sid in (0, 2, 3, 4, 1):
            tok = int(rng.integers(0, 30000))
            got = nat.append(sid, tok)
            assert got == ref.append(sid, tok)
            slot, src, dst = got
            if src >= 0:
                copy(src, dst)
                copies += 1
            write([slot], _bf16(rng, (1, HKV, D)), _bf16(rng, (1, HKV, D)))
    assert copies == 3                            # samples 0, 2, 3 copy; 4 writes in place

    live = [0, 1, 2, 3, 4, 7]
    width = 16
    tab, lens = nat.tables(live, width)
    assert tab.tolist() == [ref.table(s, width) for s in live]
    assert np.array_equal(k_dev.view(torch.int16).cpu().numpy().view(np.uint16), k_host)
    assert np.array_equal(v_dev.view(torch.int16).cpu().numpy().view(np.uint16), v_host)

    q = _bf16(rng, (len(live), HKV * G, D))
    out = torch.empty((len(live), HKV * G, D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / np.sqrt(D)
    pa.pa_decode(out, torch_from_storage(q, "bf16"), k_dev, v_dev, torch.from_numpy(tab).cuda(),
                 torch.from_numpy(lens).cuda(), int(lens.max()), scale)
    torch.cuda.synchronize()
    want = oracle.decode_ref(q, k_host, v_host, tab, lens, scale, q_kind="bf16", kv_kind="bf16")
    err = max_abs_err(as_f64(out), want)
    print(f"manager-driven decode: lens={lens.tolist()} copies={copies} max_abs_err={err:.3e}")
    assert err <= TOL["bf16"]
