"""Softmax scales other than 1/sqrt(D) on the GPU (the C ABI takes any finite one).

A negative scale reverses the ranking of the scores, zero makes the weights
uniform over the attended tokens, and a large one makes them nearly one-hot.
Each is checked against the fp64 oracle run with the same scale, for plain
decode (fixed and balanced splits), 4 drafts and prefill chunks of 16, 40 and
100 tokens, BF16 and FP8.  Bars: mean-abs 1e-3 everywhere, and per element max-abs 1e-2
against the fp64 oracle -- except where the output's own BF16 step is coarser
than that bar: with the sharp scale an output is close to one V row (|o| up to
about 4), and one BF16 ulp is 2^-6 for |o| in [2, 4) and 2^-5 in [4, 8), so
even the correctly rounded oracle is up to half of that away from it.  There
an element passes within one BF16 ulp of bf16_RNE(oracle).
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from oracle import bf16_from_f32_rne, bf16_to_f64, oracle_decode, oracle_decode_multi
from tests.oracle_fill import oracle_fill
from tests.test_gpu_parity import MAX_ABS, MEAN_ABS, log, out_f64

pytestmark = pytest.mark.gpu

SCALES = (-1.0, 0.0, 4.0)   # multiples of the workload's own 1/sqrt(D)


def bf16_ulp(y):
    """One BF16 ulp at the values y (BF16 values, fp64): 2^(floor(log2|y|) - 7)."""
    a = np.abs(y)
    return np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)


def _check(got, ref, what, sharp):
    e = np.abs(got - ref)
    log("%s: max-abs %.3g mean-abs %.3g" % (what, e.max(), e.mean()))
    assert np.all(np.isfinite(got))
    assert e.mean() <= MEAN_ABS, e.mean()
    rounded = bf16_to_f64(bf16_from_f32_rne(ref.astype(np.float32)))
    ulp = bf16_ulp(rounded)
    ok = (e <= MAX_ABS) | ((ulp > MAX_ABS) & (np.abs(got - rounded) <= ulp))
    assert ok.all(), (e[~ok][:4], ref[~ok][:4])
    if not sharp:
        assert e.max() <= MAX_ABS, e.max()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_scales(kv):
    w = make_workload(2, batch=4, lens=[1, 300, 1500, 4097], kv=kv, stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    cache, _ = oracle_fill(w)
    for f in SCALES:
        sigma = float(np.float32(w.sigma * f))
        ref = oracle_decode(cache, w.q, w.block_table, w.lens, sigma)
        for parts in (0, 1, 5):
            out = pa.decode(dw.cache, dw.q, dw.block_table, dw.lens, sigma, num_partitions=parts)
            torch.cuda.synchronize()
            _check(out_f64(out), ref, "%s decode scale %gx partitions %d" % (kv, f, parts),
                   sharp=f > 1)


# 4 drafts; prefill chunks of 16 tokens (64 columns: one multi-query wave per
# unit) and of 40 and 100 tokens (160 and 400 columns: the page-sharing kernel,
# which applies the scale inside the exponential and takes the column extreme
# from the raw scores, so the sign and zero of the scale are its own cases)
@pytest.mark.parametrize("kv,T", [("fp8", 4), ("bf16", 16), ("bf16", 40), ("fp8", 100)])
def test_multi_query_and_prefill_scales(kv, T):
    w = make_workload(2, batch=3, lens=[max(20, T + 20), 700, 2100], q_len=T, kv=kv,
                      stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    cache, _ = oracle_fill(w)
    run = pa.decode_multi if T <= 8 else pa.prefill
    for f in SCALES:
        sigma = float(np.float32(w.sigma * f))
        ref = oracle_decode_multi(cache, w.q, w.block_table, w.lens, sigma)
        out = run(dw.cache, dw.q, dw.block_table, dw.lens, sigma)
        torch.cuda.synchronize()
        _check(out_f64(out), ref, "%s T=%d scale %gx" % (kv, T, f), sharp=f > 1)
