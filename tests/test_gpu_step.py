"""pa_decode_step (a decode step's append and decode in one call) on the GPU.

The step's append runs in the same launch as the decode's validation and split
plan.  Its pages, scales, outputs and flags must be those of pa_cache_append
followed by pa_decode / pa_decode_multi, bit for bit; the outputs are also
checked against the fp64 oracle with the bars of the other parity tests
(max-abs 1e-2, mean-abs 1e-3, flags bit-exact, flagged rows +0.0).
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from tests.oracle_fill import oracle_sequences_parallel
from tests.test_gpu_parity import compare_outputs, compare_pools, expected_flags, flags_of, log

pytestmark = pytest.mark.gpu


def _state(cache):
    """The cache's bytes: pools, and FP8 scales as raw bits (NaN-safe)."""
    ts = [cache.k, cache.v] + [t for t in (cache.k_scale, cache.v_scale) if t is not None]
    return [t.contiguous().view(torch.uint8).clone() for t in ts]


def _restore(cache, snap):
    ts = [cache.k, cache.v] + [t for t in (cache.k_scale, cache.v_scale) if t is not None]
    for t, s in zip(ts, snap):
        t.view(torch.uint8).copy_(s)


@pytest.mark.parametrize("cfg,kw,parts", [
    (1, {}, 0),                                                        # BF16, D 64, one partition
    (3, dict(batch=4, lens=[100, 2000, 4097, 9000]), 4),               # FP8, stale tags, split-K 4
    (3, dict(batch=4, lens=[17, 33, 4096, 5000], stale_frac=0.0), 0),  # fresh pages, balanced split
    (4, dict(batch=2), 0),                                             # HEAD layout, ragged heads
    (2, dict(lens=np.array([[40, 1, 700, 16, 17, 3001, 0, 64], [5, 900, 33, 2000, 1, 48, 300, 15]]),
             kv="fp8", layout="head", stale_frac=0.02), 0),                       # HEAD FP8
    (2, dict(batch=3, lens=[40, 700, 3000], q_len=4), 0),              # 4 drafts
    (3, dict(batch=3, lens=[9, 300, 2049], q_len=8, stale_frac=0.0), 0),   # 8 drafts, FP8
])
def test_step_matches_append_then_decode(cfg, kw, parts):
    w = make_workload(cfg, **kw)
    log("step: workload %d B=%d layout=%s kv=%s T=%d parts=%d" % (
        cfg, w.B, w.layout, w.kv_dtype, w.q_len, parts))
    dw = build_device_workload(w)
    before = _state(dw.cache)
    dw.step_append()
    ref = dw.decode(check=True, num_partitions=parts).clone()
    torch.cuda.synchronize()
    ref_flags = dw.flags.clone()
    ref_state = _state(dw.cache)
    _restore(dw.cache, before)
    dw.flags.fill_(-1)
    out = dw.decode_step(check=True, num_partitions=parts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dw.flags, ref_flags)
    for got, want in zip(_state(dw.cache), ref_state):
        assert torch.equal(got, want)


@pytest.mark.parametrize("cfg,kw", [
    (3, dict(batch=6, lens=[1, 16, 17, 500, 4097, 12000], stale_frac=0.0)),
    (3, dict(batch=5, lens=[20, 300, 700, 2000, 5000])),               # stale tags: flags
    (2, dict(batch=3, lens=[8, 900, 2500], q_len=4, kv="fp8")),
])
def test_step_against_oracle(cfg, kw):
    w = make_workload(cfg, **kw)
    log("step vs oracle: workload %d B=%d kv=%s T=%d" % (cfg, w.B, w.kv_dtype, w.q_len))
    dw = build_device_workload(w)
    out = dw.decode_step(check=True)
    torch.cuda.synchronize()
    fl = flags_of(dw)
    assert np.array_equal(fl, expected_flags(w)), fl
    seqs = list(range(w.B))
    ora = oracle_sequences_parallel(w, seqs)
    compare_pools(dw, ora, seqs)
    compare_outputs(out, ora, seqs, fl, "step")


def test_step_without_new_tokens_is_the_decode():
    w = make_workload(2, batch=3, lens=[50, 600, 1500], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    ref = dw.decode(check=True).clone()
    before = _state(dw.cache)
    zero = torch.zeros_like(dw.n_step)
    k0 = dw.k_step[:, :, :0].contiguous()
    out = pa.decode_step(dw.cache, dw.q, dw.block_table, dw.lens, zero, k0, k0, dw.lens, w.sigma,
                         expected_tags=dw.expected_tags, flags=dw.flags)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    for got, want in zip(_state(dw.cache), before):
        assert torch.equal(got, want)


def test_step_full_size_matches_append_then_decode():
    """The 70B-shaped FP8 layer at full size (64 x 32K tokens, split-K 8, tag check
    on), the benchmark's step: pa_decode_step against the two calls, bit for bit
    (pools, scales, outputs, flags); the two calls are checked against the oracle
    at this size in test_gpu_parity.py."""
    w = make_workload(5)
    dw = build_device_workload(w, log=log)
    before = _state(dw.cache)
    dw.step_append()
    ref = dw.decode(check=True, num_partitions=8).clone()
    torch.cuda.synchronize()
    ref_flags = dw.flags.clone()
    ref_state = _state(dw.cache)
    _restore(dw.cache, before)
    del before
    out = dw.decode_step(check=True, num_partitions=8)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dw.flags, ref_flags)
    for got, want in zip(_state(dw.cache), ref_state):
        assert torch.equal(got, want)
