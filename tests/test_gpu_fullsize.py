"""Full-size configurations in the launch configuration the bench times: every output
element of every sequence against the oracle, and both pools bit for bit after the step's
copy-on-write copies and slot writes."""
import numpy as np
import pytest

import workload as wl
from gpu_harness import (TOL, as_f64, gpu_step, max_abs_err, oracle_decode,
                         oracle_pools_after_step, storage_bits, to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_full_size(idx):
    w = wl.make(idx)
    print(f"config {idx} {w.name}: B={w.batch} tokens={w.total_tokens} "
          f"kv_bytes={w.kv_bytes}", flush=True)
    d = to_device(w)
    out = as_f64(gpu_step(w, d, partition_size=w.partition_size))
    assert np.isfinite(out).all()
    k, v = oracle_pools_after_step(w)
    # the step's copies and writes landed bit-exactly (the untouched blocks too)
    for name, pool in (("k", k), ("v", v)):
        bits = storage_bits(d[name])
        assert np.array_equal(bits, pool.view(bits.dtype)), f"{name} pool differs"
    del d
    ref = oracle_decode(w, k, v)
    err = max_abs_err(out, ref)
    print(f"  all {w.batch} sequences: max_abs_err={err:.3e} (bar {TOL[w.kv_dtype]:g})",
          flush=True)
    assert err <= TOL[w.kv_dtype]
