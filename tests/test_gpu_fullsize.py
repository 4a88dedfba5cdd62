"""Full-size configurations in the launch configuration the bench times, checked on a
sample of sequences the oracle computes one by one (shortest, longest, seeded picks)."""
import numpy as np
import pytest

import workload as wl
from gpu_harness import (TOL, as_f64, gpu_step, max_abs_err, oracle_decode,
                         oracle_pools_after_step, sample_seqs, storage_bits, to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size_sampled(idx):
    w = wl.make(idx)
    print(f"config {idx} {w.name}: B={w.batch} tokens={w.total_tokens} "
          f"kv_bytes={w.kv_bytes}", flush=True)
    d = to_device(w)
    out = as_f64(gpu_step(w, d, partition_size=w.partition_size))
    assert np.isfinite(out).all()
    seqs = sample_seqs(w, n=6)
    if w.slot_mapping is not None or w.copy_pairs is not None:
        k, v = oracle_pools_after_step(w)
        # the step's writes landed bit-exactly
        assert np.array_equal(storage_bits(d["k"]), k.view(storage_bits(d["k"]).dtype))
    else:
        k, v = w.k_pool, w.v_pool
    ref = oracle_decode(w, k, v, seqs=seqs)
    err = max_abs_err(out[seqs], ref)
    print(f"  sampled {len(seqs)} sequences: max_abs_err={err:.3e}", flush=True)
    assert err <= TOL[w.kv_dtype]
