"""Chunked prefill over the paged cache on the GPU against the oracle.

The chunk's C tokens are the last C tokens of each unit; token t sees tokens
0 .. L - C + t (oracle_decode_multi, pinned in test_oracle_multi.py).  Same
bars as decode: BF16 outputs within max-abs 1e-2 / mean-abs 1e-3 of the fp64
oracle, flags bit-exact, flagged rows +0.0.  Chunks of more than 64 columns
run on the page-sharing kernel: 32-column blocks, four per workgroup, sharing
each page through LDS; the cases include workgroups whose last blocks lie past
the unit's columns (132 and 291 columns: 3 and 2 of 4 waves without columns),
both layouts and dtypes, D 64, G up to 16, split prefixes, a prefix of zero,
and sampled checks at a realistic size (BF16 and FP8 caches).
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from oracle import attention_f64, bf16_to_f64, gather_unit
from tests.oracle_fill import oracle_fill
from tests.test_gpu_parity import MAX_ABS, MEAN_ABS, log, out_f64, run_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,kw,C,parts", [
    (1, dict(lens=[40, 100, 300, 511]), 33, (0, 1, 3)),           # D 64, 3 column blocks
    (2, dict(batch=3, lens=[256, 1500, 4000]), 256, (0, 1, 4)),   # 16 column blocks, BF16
    (3, dict(batch=2, lens=[300, 2000], stale_frac=0.02), 128, (0, 2)),   # FP8, stale tags
    (1, dict(lens=[40, 64, 300, 511], heads=(16, 1)), 40, (0, 2)),        # G 16, Hkv 1
    (2, dict(batch=2, lens=[100, 700], heads=(24, 8)), 97, (0, 3)),       # G 3: ragged blocks
    (2, dict(lens=np.array([[80, 300, 700, 1000, 90, 2000, 65, 64], [64, 100, 4000, 70, 99, 640, 300, 1000]]),
             kv="fp8", layout="head"), 64, (0, 2)),                       # FP8, HEAD
    (2, dict(batch=2, lens=[200, 1500], kv="fp8", head_dim=64), 100, (0, 2)),   # FP8, D 64
    (2, dict(lens=np.array([[80, 700, 64, 1300, 99, 333, 65, 400], [1000, 64, 257, 90, 2048, 71, 640, 128]]),
             kv="fp8", layout="head", head_dim=64), 48, (0, 3)),             # FP8, HEAD, D 64
])
def test_prefill_matches_oracle(cfg, kw, C, parts):
    w = make_workload(cfg, q_len=C, **kw)
    run_case(w, partitions=parts)


def test_prefill_headwise():
    lens = np.array([[64, 100, 512, 64, 65, 130, 999, 64], [2048, 80, 4096, 70, 64, 640, 3000, 1000]])
    w = make_workload(4, lens=lens, q_len=64)
    run_case(w, partitions=(0, 16))


def test_prefill_many_units_keep_index_order():
    """More than 64 lengths (72 HEAD units): the launch keeps the index order
    instead of starting the longest units first."""
    lens = np.random.default_rng(7).integers(64, 700, size=(9, 8))
    w = make_workload(4, lens=lens, q_len=64)
    run_case(w, partitions=(0,))


def test_prefill_short_chunks_equal_decode_multi_and_decode():
    w = make_workload(2, batch=3, lens=[9, 600, 2000], q_len=4)
    dw = build_device_workload(w)
    dw.step_append()
    a = pa.decode_multi(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, num_partitions=4)
    b = pa.prefill(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, num_partitions=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    q1 = dw.q[:, -1:].contiguous()
    c = pa.prefill(dw.cache, q1, dw.block_table, dw.lens, w.sigma, num_partitions=2)
    d = pa.decode(dw.cache, q1[:, 0].contiguous(), dw.block_table, dw.lens, w.sigma, num_partitions=2)
    torch.cuda.synchronize()
    assert torch.equal(c[:, 0].view(torch.int16), d.view(torch.int16))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_realistic_size_sampled(kv):
    """Llama-3.1-8B-shaped layer (BF16 or FP8 cache), 4 sequences with prefixes 0, 2K,
    8K, 30K and a 2048-token chunk: sampled rows against the oracle, all rows finite.
    (FP8: the page-sharing kernel widens each page once per workgroup, over 256-page
    id segments.)"""
    C = 2048
    prefix = np.array([0, 2048, 8192, 30720])
    w = make_workload(2, batch=4, lens=prefix + C, q_len=C, table_width=2048, kv=kv)
    dw = build_device_workload(w, log=log)
    dw.step_append()
    out = pa.prefill(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma,
                     expected_tags=dw.expected_tags, flags=dw.flags)
    torch.cuda.synchronize()
    assert np.all(dw.flags.cpu().numpy() == 0)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    cache, _ = oracle_fill(w, seqs=[0, 3])
    errs = []
    for b in (0, 3):
        L = int(w.lens[b])
        for h in (0, 5):
            K, V = gather_unit(cache, w.block_table[b], h, L)
            for t in (0, 1, 777, C - 1):
                n = L - C + t + 1
                for g in (0, w.G - 1):
                    hq = h * w.G + g
                    ref, _ = attention_f64(bf16_to_f64(w.q[b, t, hq]), K[:n], V[:n], w.sigma)
                    errs.append(np.abs(got[b, t, hq] - ref))
    e = np.concatenate(errs)
    log("prefill sampled (%s): max-abs %.3g mean-abs %.3g over %d values" % (kv, e.max(), e.mean(), e.size))
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS
