"""The 70B-shaped FP8 decode layer at full size on the GPU, every sequence
against the oracle: B 64, 64 query / 8 KV heads, D 128, 32768 tokens each
(4.29 GB of FP8 KV; "Cloudflare quantizes Kimi and GLM caches for 41% faster
inference", KV cache quantization paragraph: the FP8 cache for the
memory-bound decode).

One cache fill and one oracle pass (in chunks of 16 sequences) serve every
check at this size:
  - pool bytes and FP8 scales of all 131,072 pages, bit for bit;
  - flags, and all 4,096 output rows at split-K 8 (the benchmark's launch
    configuration) and with the automatic split (max-abs 1e-2, mean-abs 1e-3);
  - pa_decode_step (the benchmark's step) against pa_cache_append then
    pa_decode: pools, scales, outputs and flags bit for bit;
  - the scored decode (eviction scores): outputs bitwise those of pa_decode,
    every read score slot against the oracle's attention mass, every other
    slot unchanged.
The multi-query steps at this size are in tests/test_gpu_multi.py.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from tests.oracle_fill import oracle_chunks
from tests.test_gpu_evict import RTOL, ATOL, _expected_scores, _read_slots
from tests.test_gpu_parity import (
    compare_outputs,
    compare_pools,
    expected_flags,
    flags_of,
    log,
    logical_pools,
)
from tests.test_gpu_step import _restore, _state

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_workload5_full():
    w = make_workload(5)
    dw = build_device_workload(w, log=log)
    before = _state(dw.cache)
    dw.step_append()
    outs = {}
    for p in (8, 0):
        outs[p] = dw.decode(check=True, num_partitions=p).clone()
        torch.cuda.synchronize()
        fl = flags_of(dw)
        assert np.array_equal(fl, expected_flags(w)), fl
    log("decode done; the fused step against the two calls")
    ref_state = _state(dw.cache)
    _restore(dw.cache, before)
    del before
    dw.flags.fill_(-1)
    out_step = dw.decode_step(check=True, num_partitions=8)
    torch.cuda.synchronize()
    assert torch.equal(out_step.view(torch.int16), outs[8].view(torch.int16))
    assert np.array_equal(flags_of(dw), fl)
    for got, want in zip(_state(dw.cache), ref_state):
        assert torch.equal(got, want)
    del ref_state, out_step
    log("scored decode")
    rng = np.random.default_rng(5)
    read = _read_slots(w, list(range(w.B)))
    bn = rng.random(dw.cache.new_scores().shape).astype(np.float32)
    bn[read & (rng.random(bn.shape) < 0.5)] = 0.0    # zero priors make the mass itself visible
    scores = torch.from_numpy(bn).cuda()
    out_s = pa.decode_scored(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, scores,
                             expected_tags=dw.expected_tags, flags=dw.flags, num_partitions=8)
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), outs[8].view(torch.int16))
    got_scores = scores.cpu().numpy()
    assert np.array_equal(got_scores[~read], bn[~read])
    del scores, out_s
    logical = logical_pools(dw)
    for part in oracle_chunks(w, range(w.B), 16, with_mass=True):
        seqs = sorted(part)
        compare_pools(dw, part, seqs, logical)
        for p in (8, 0):
            compare_outputs(outs[p], part, seqs, fl,
                            "sequences %d..%d partitions=%d" % (seqs[0], seqs[-1], p))
        exp = _expected_scores(w, part, seqs, 1, bn)
        mine = _read_slots(w, seqs)
        d = got_scores[mine].astype(np.float64) - exp[mine]
        inc = exp[mine] - bn[mine]
        assert np.all(np.abs(d) <= RTOL * inc + ATOL + 2 ** -23 * np.abs(exp[mine])), \
            np.abs(d).max()
        log("checked sequences %d..%d (scores: max rel err %.3g)" % (
            seqs[0], seqs[-1], (np.abs(d) / np.maximum(inc, 1e-30)).max()))
