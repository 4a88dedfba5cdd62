"""pa_decode_noalloc (the allocation-free decode, for callers that cannot allocate) through
the C ABI against pa_decode on the same inputs: the same kernels with the workspace in the
library's static scratch instead of the caller's buffer, so the outputs must be the same
bits. Two calls in a row, the second with a smaller input, so the second runs on the
scratch contents the first left behind; each output is also checked against the oracle."""
import numpy as np
import pytest

import workload as wl
from gpu_harness import TOL, as_f64, gpu_decode, max_abs_err, oracle_decode, to_device

pytestmark = pytest.mark.gpu


def _noalloc(w, d, part):
    import torch
    import paged_kv_cache_367_amd as pa
    out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.bfloat16, device="cuda")
    pa.pa_decode_noalloc(out, d["q"], d["k"], d["v"], d["tables"], d["lens"],
                         w.max_context_len, w.scale, w.k_scale, w.v_scale,
                         partition_size=part)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_pa_decode_on_two_calls():
    import paged_kv_cache_367_amd as pa
    cases = [
        # fp8 long context with 512-token partitions (the merge over many pieces), then
        wl.make(5, batch=3),
        # a smaller bf16 GQA batch under the default split (the per-chunk merge)
        wl.make(3, batch=20, len_range=(16, 1500)),
    ]
    sizes = []
    for w in cases:
        part = w.partition_size
        d = to_device(w)
        desc = pa.binding.make_desc(d["q"], d["k"], d["tables"], None, part)
        need = pa.pa_decode_workspace_bytes(desc, w.max_context_len)
        assert 0 < need <= 64 << 20
        sizes.append(need)
        ref_out = as_f64(gpu_decode(w, d, partition_size=part))     # caller's workspace
        got = as_f64(_noalloc(w, d, part))
        assert np.array_equal(got, ref_out), f"{w.name}: differs from pa_decode"
        err = max_abs_err(got, oracle_decode(w))
        print(f"{w.name}: workspace {need} B, partition {part}: bitwise equal to pa_decode, "
              f"max_abs_err vs oracle {err:.3e}", flush=True)
        assert err <= TOL[w.kv_dtype]
    assert sizes[1] < sizes[0]
