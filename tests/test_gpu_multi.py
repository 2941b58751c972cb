"""Multi-query decode (speculative verification) on the GPU against the oracle.

Query token t of T sits at position L - T + t and sees tokens 0 .. L - T + t.
Same bars as plain decode: pool bytes, scales and flags bit-exact; BF16
outputs within max-abs 1e-2 / mean-abs 1e-3 of the fp64 oracle; rows of
flagged sequences and of tokens with nothing to attend exactly +0.0.  The
cases cover every column-tile count of the kernel (G * T up to 16, 32, 64),
both layouts and dtypes, drafts split by a partition boundary, and lengths
shorter than T.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from oracle import oracle_decode_multi, oracle_validate
from tests.oracle_fill import oracle_fill
from tests.test_gpu_parity import (
    MAX_ABS,
    MEAN_ABS,
    compare_outputs,
    flags_of,
    log,
    out_f64,
    run_case,
    run_full_case,
)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_multi_tiny_every_qlen(T):
    """BF16, D 64, G 4: T 2-3 fit one column tile, 5 and 8 take two."""
    w = make_workload(1, q_len=T)
    run_case(w, partitions=(0, 2, 32))


def test_multi_one_token_is_decode_bitwise():
    w = make_workload(2, batch=4, lens=[1, 40, 700, 3000])
    dw = build_device_workload(w)
    dw.step_append()
    a = dw.decode(num_partitions=4)
    b = pa.decode_multi(dw.cache, dw.q[:, None].contiguous(), dw.block_table, dw.lens, w.sigma,
                        expected_tags=dw.expected_tags, flags=dw.flags, num_partitions=4)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b[:, 0].view(torch.int16))


def test_multi_bf16_ragged_and_partition_boundary_inside_drafts():
    """L = 1030, T = 8: with 64 partitions of 128 tokens the drafts 1022..1029
    straddle the boundary at 1024, so the first drafts see an empty partition."""
    w = make_workload(2, batch=5, lens=[8, 17, 300, 1030, 4096], q_len=8)
    run_case(w, partitions=(0, 1, 3, 8, 64))


@pytest.mark.parametrize("layout,D,T", [("head", 128, 3), ("head", 64, 8), ("seq", 64, 5)])
def test_multi_fp8_other_formats(layout, D, T):
    if layout == "head":
        lens = np.array([[8, 300, 17, 2049, 9, 100, 1000, 64], [4096, 12, 650, 33, 8, 700, 64, 90]])
    else:
        lens = [8, 300, 2049, 5000]
    w = make_workload(2, lens=lens, kv="fp8", layout=layout, head_dim=D, q_len=T, stale_frac=0.0)
    run_case(w, partitions=(0, 2))


def test_multi_fp8_stale_tags():
    w = make_workload(3, batch=5, lens=[5, 700, 2049, 5000, 9000], q_len=5, stale_frac=0.02)
    assert w.stale.any()
    run_case(w, partitions=(0, 4, 16))


def test_multi_headwise():
    lens = np.array([[33, 8, 512, 16, 17, 100, 9, 64], [2048, 8, 4096, 4097, 15, 16, 31, 1000]])
    w = make_workload(4, lens=lens, q_len=8)
    run_case(w, partitions=(0, 16, 64))


@pytest.mark.parametrize("cfg,heads,T,kw", [
    (1, (16, 1), 4, {}),                                         # D 64, 64 columns, Hkv 1
    (1, (8, 4), 8, {}),                                          # Hkv 4: XCD order, G 2
    (5, None, 8, dict(batch=3, lens=[40, 3000, 9000])),          # FP8 D 128, 64 columns
    (5, None, 4, dict(batch=3, lens=[4, 1111, 5000])),           # FP8 D 128, 32 columns
    (2, (24, 8), 7, dict(batch=3, lens=[7, 600, 2500])),         # G 3: 21 columns, two tiles
])
def test_multi_column_tiles(cfg, heads, T, kw):
    w = make_workload(cfg, q_len=T, heads=heads, **kw)
    run_case(w, partitions=(0, 1, 8))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [4, 8])
def test_multi_workload5_full(T):
    """70B-shaped FP8 cache, L = 32768, T = 4 or 8 drafts (32 or 64 columns per
    unit), all 64 sequences against the oracle: the automatic split the
    benchmark times (split-K 4) and split-K 8; the pages of the T-token
    append (re-quantised where the drafts raise a page's scale) bit for bit."""
    run_full_case(make_workload(5, q_len=T), partitions=(0, 8), pools=(T == 8))


def test_multi_lengths_shorter_than_the_drafts():
    """Decode with lengths below T: tokens before position 0 get +0.0 rows."""
    w = make_workload(1, q_len=4)
    dw = build_device_workload(w)
    dw.step_append()
    cache, _ = oracle_fill(w)
    lens = np.array([2, 0, 4, 511], np.int32)
    lens_d = torch.from_numpy(lens).to("cuda")
    for parts in (0, 1, 8):
        out = pa.decode_multi(dw.cache, dw.q, dw.block_table, lens_d, w.sigma,
                              expected_tags=dw.expected_tags, flags=dw.flags, num_partitions=parts)
        torch.cuda.synchronize()
        fl = flags_of(dw)
        want_fl = oracle_validate(w.layout, w.P, w.S, w.block_table, lens, w.page_tags,
                                  w.expected_tags, w.W)
        assert np.array_equal(fl, want_fl)
        ref = oracle_decode_multi(cache, w.q, w.block_table, lens, w.sigma, flags=fl)
        got = out_f64(out)
        assert np.all(got[0, :2] == 0) and np.all(got[1] == 0)      # nothing to attend
        assert np.all(out[0, :2].view(torch.int16).cpu().numpy() == 0)  # +0.0, not -0.0
        e = np.abs(got - ref)
        log("short lengths, partitions=%d: max-abs %.3g" % (parts, e.max()))
        assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS
        assert np.all(np.isfinite(got))


def test_multi_graph_replays_match_eager():
    w = make_workload(3, batch=4, lens=[100, 2000, 4097, 9000], q_len=6, stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    eager = dw.decode(num_partitions=4).clone()
    g = pa.DecodeStepGraph(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step, dw.v_step,
                           dw.q, dw.lens, w.sigma, expected_tags=dw.expected_tags, flags=dw.flags,
                           num_partitions=4)
    for i in range(3):
        out = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        _ = dw.decode(check=False, num_partitions=4)
        torch.cuda.synchronize()
    ora = {b: {"out": r} for b, r in
           enumerate(oracle_decode_multi(oracle_fill(w)[0], w.q, w.block_table, w.lens, w.sigma))}
    compare_outputs(out, ora, range(w.B), flags_of(dw), "graph")
