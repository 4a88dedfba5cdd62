"""Decode rows that attend over a handful of tokens, where the weights' rounding counts
most (intelliparadigm article, section 5.1: check masks at block boundaries and the
error half precision accumulates).

256 sequences per case with lengths drawn from [2, 48] (one to three blocks, every
ragged tail), for every 16-bit and fp8 cache, group size 1, 4 and 8, head_dim 64 and 128,
two seeds; every output element is compared with the fp64 oracle.

Output rounding sets the floor: the output is in q's dtype, and rounding the oracle's own
result to that dtype already moves it by up to half an ulp of |out| (bf16: 2^-9 |out|,
about 7.8e-3 for |out| in [2, 4), which rows over two or three tokens reach). The test
prints that floor next to the GPU's error and checks that the bar stays above it at these
inputs. With an fp32 output only the kernel's own arithmetic is left: the softmax weights
enter the matrix cores as a hi and a lo 16-bit part (within 2^-16 of the fp32 weight), so
the error is a few 1e-5 at most; 2e-3 is the bar.
"""
import numpy as np
import pytest

import workload as wl
from gpu_harness import TOL, as_f64, gpu_decode, max_abs_err, oracle_decode, to_device

pytestmark = pytest.mark.gpu

FP32_OUT_TOL = 2e-3
CASES = [(kv, G, d) for kv in ("bf16", "f16", "fp8_e4m3") for G in (1, 4, 8) for d in (64, 128)]


def few_token_workload(kv, G, d, seed, batch=256):
    rng = np.random.default_rng(1000 * G + d + seed)
    lens = rng.integers(2, 49, size=batch)
    return wl.custom(batch=batch, num_q_heads=2 * G, num_kv_heads=2, head_dim=d, kv_dtype=kv,
                     context_lens=lens, seed=5000 + 100 * G + d + seed)


def output_rounding_floor(ref: np.ndarray, kind: str) -> float:
    """Largest change rounding the oracle's result to the output dtype makes."""
    import torch
    t = torch.from_numpy(ref)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[kind]
    return float((t.to(dt).double() - t).abs().max())


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("kv,G,d", CASES)
def test_few_token_rows(kv, G, d, seed):
    w = few_token_workload(kv, G, d, seed)
    dev = to_device(w)
    ref = oracle_decode(w)
    err = max_abs_err(as_f64(gpu_decode(w, dev)), ref)
    err32 = max_abs_err(as_f64(gpu_decode(w, dev, out_dtype="f32")), ref)
    floor = output_rounding_floor(ref, w.out_dtype)
    bar = TOL[kv]
    print(f"{kv} G={G} d={d} seed={seed}: max|out|={np.abs(ref).max():.3f} "
          f"err({w.out_dtype} out)={err:.3e} [rounding floor {floor:.3e}, bar {bar:g}, "
          f"margin {bar / max(err, 1e-30):.2f}x] err(f32 out)={err32:.3e} "
          f"[bar {FP32_OUT_TOL:g}, margin {FP32_OUT_TOL / max(err32, 1e-30):.0f}x]", flush=True)
    assert floor < bar, "inputs whose own output rounding exceeds the bar"
    assert err <= bar
    assert err32 <= FP32_OUT_TOL


@pytest.mark.parametrize("kv", ["bf16", "f16", "fp8_e4m3"])
@pytest.mark.parametrize("part", [16, 32])
def test_few_token_rows_cut_into_pieces(kv, part):
    """The same rows with every block (part = 16) or pair of blocks (32) a split-KV
    partition of its own, so that the merge combines one-block pieces."""
    w = few_token_workload(kv, 4, 128, 7, batch=96)
    ref = oracle_decode(w)
    out = as_f64(gpu_decode(w, to_device(w), partition_size=part, out_dtype="f32"))
    err = max_abs_err(out, ref)
    print(f"{kv} partition {part}: err(f32 out)={err:.3e}", flush=True)
    assert err <= FP32_OUT_TOL
