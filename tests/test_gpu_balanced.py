"""The length-balanced split of the automatic decode on the GPU.

With num_partitions = 0 and a table wider than 32 pages, the chunk size comes
from the real lengths, on the device: a unit then has no partition (nothing to
attend), one (its output rows are written by the attention kernel itself) or
several (merged by the reduce).  Same bars as the other parity tests: BF16
outputs within max-abs 1e-2 / mean-abs 1e-3 of the fp64 oracle, flags
bit-exact, flagged and empty rows +0.0; plus bitwise run-to-run determinism.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from tests.oracle_fill import oracle_sequences_parallel
from tests.test_gpu_parity import compare_outputs, flags_of, log, run_case

pytestmark = pytest.mark.gpu


def _balanced_case(w, flag=(), seqs=None):
    """Auto decode against the oracle, with stale expected tags planted on `flag`."""
    log("balanced: workload %d (%s) B=%d layout=%s W=%d lens[:6]=%s" % (
        w.cfg_id, w.name, w.B, w.layout, w.W, w.lens.ravel()[:6].tolist()))
    dw = build_device_workload(w, log=log)
    dw.step_append()
    for b in flag:
        dw.expected_tags[b].view(-1)[0] ^= 1
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    ora = oracle_sequences_parallel(w, [b for b in seqs if b not in flag])
    out = dw.decode(check=True, num_partitions=0).clone()
    again = dw.decode(check=True, num_partitions=0)
    torch.cuda.synchronize()
    fl = flags_of(dw)
    assert all(fl[b] != 0 for b in flag) and all(fl[b] == 0 for b in range(w.B) if b not in flag)
    compare_outputs(out, ora, [b for b in seqs if b not in flag], fl, "balanced")
    for b in flag:
        assert np.all(out[b].view(torch.int16).cpu().numpy() == 0)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "not deterministic"
    return dw, out


def test_all_units_empty():
    w = make_workload(2, batch=3, lens=[0, 0, 0], table_width=64)
    dw = build_device_workload(w)
    dw.step_append()
    out = dw.decode(check=True, num_partitions=0)
    torch.cuda.synchronize()
    assert pa.num_partitions(dw.cache, dw.block_table, dw.lens, w.Hq) == 0   # balanced
    assert np.all(out.view(torch.int16).cpu().numpy() == 0)


def test_one_long_unit_among_short_ones_and_flags():
    # sequence 0 spans many partitions; the short ones get one each (written
    # directly); sequence 1 (several partitions) and 4 (one) are aborted
    lens = [8000, 6000, 20, 1, 300, 0, 17, 64]
    w = make_workload(2, batch=8, lens=lens, table_width=512)
    _balanced_case(w, flag=(1, 4))


def test_headwise_ragged_heads():
    lens = np.array([[4096, 1, 17, 600, 0, 2048, 33, 16], [5, 3000, 1000, 16, 17, 64, 4095, 1]])
    _balanced_case(make_workload(4, lens=lens, table_width=256), flag=(1,))


@pytest.mark.parametrize("layout_cfg", [1, 4])
def test_two_kv_heads_plain_order(layout_cfg):
    # Hkv = 2: no XCD-aware order; SEQ pairs hold two heads, HEAD pairs one
    if layout_cfg == 1:
        w = make_workload(1, batch=6, lens=[700, 1, 64, 2000, 33, 0], table_width=128)
    else:
        lens = np.array([[700, 1], [64, 2000], [33, 0], [1500, 16]])
        w = make_workload(4, lens=lens, heads=(8, 2), table_width=128)
    _balanced_case(w)


def test_more_than_1024_groups():
    # 1100 sequences (groups): the planner scans its partition counts in
    # several tiles of 1024; a sample of sequences is checked against the oracle
    rng = np.random.default_rng(11)
    lens = rng.integers(0, 700, size=1100).astype(np.int32)
    lens[[3, 1050]] = 2047                    # long ones on both sides of the tile edge
    w = make_workload(1, batch=1100, lens=lens, table_width=128)
    _balanced_case(w, seqs=[0, 1, 3, 500, 1023, 1024, 1050, 1099])


@pytest.mark.parametrize("cfg", [2, 4])
def test_multi_query_balanced(cfg):
    # SEQ (pairs of 8 heads) and HEAD (one head per pair; slots by unit)
    if cfg == 2:
        w = make_workload(2, batch=5, lens=[4, 9, 3000, 700, 8000], q_len=4, table_width=512)
    else:
        lens = np.array([[4, 2000, 9, 700, 4096, 5, 64, 33], [3000, 4, 17, 8, 1000, 4095, 16, 250]])
        w = make_workload(4, lens=lens, q_len=4, table_width=256)
    run_case(w, partitions=(0,))


def test_scored_balanced_matches_fixed_split():
    """Scored decode on the balanced split: the eviction scores match those of
    a fixed split to fp32 rounding (the rows' max and sum merge in another
    order), and the outputs are those of pa_decode on the same split."""
    w = make_workload(3, batch=4, lens=[40, 700, 9000, 16000], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    plain = dw.decode(num_partitions=0).clone()
    got = {}
    for p in (0, 4):
        scores = dw.cache.new_scores()
        out = pa.decode_scored(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, scores,
                               num_partitions=p)
        torch.cuda.synchronize()
        if p == 0:
            assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
        got[p] = scores.cpu().numpy().astype(np.float64)
    d = np.abs(got[0] - got[4])
    assert np.all(d <= 1e-5 * np.abs(got[4]) + 1e-12), d.max()


def test_graph_replans_when_lengths_change():
    """A captured decode step reads the lengths at every replay, so the split
    is planned anew: after the lengths change in place, a replay equals the
    eager decode of the same cache, bit for bit."""
    w = make_workload(2, batch=4, lens=[50, 600, 1500, 3000], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    g = pa.DecodeStepGraph(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step, dw.v_step,
                           dw.q, dw.lens, w.sigma, expected_tags=dw.expected_tags, flags=dw.flags)
    first = g.replay().clone()
    torch.cuda.synchronize()
    ref = dw.decode(check=True)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), ref.view(torch.int16))
    # long sequences get short, a short one grows within its last page (the
    # table holds pages for the old lengths only)
    new = torch.tensor([60, 200, 1500, 100], dtype=torch.int32, device="cuda")
    dw.lens.copy_(new)
    dw.lens_old.copy_(new - 1)
    out = g.replay().clone()             # appends at the new positions, then decodes
    torch.cuda.synchronize()
    ref = dw.decode(check=True)
    torch.cuda.synchronize()
    assert np.all(flags_of(dw) == 0)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert not torch.equal(out[3].view(torch.int16), first[3].view(torch.int16))


def _a256(x):
    return (x + 255) // 256 * 256


def _rule_chunk(pages, hpg, W, target=2048, min_chunk=32):
    """The planner's rule: the smallest chunk of at least min_chunk pages (at most
    W) whose partitions, each group's last one rounded up, make <= target waves."""
    lo = min(max(-(-int(pages.sum()) * hpg // target), min_chunk), W)
    for c in range(lo, W + 1):
        if int((-(-pages // c)).sum()) * hpg <= target:
            return c
    return W


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_plan_follows_the_rule(cfg):
    """The plan the automatic decode leaves in its workspace (layout of
    pa_decode_workspace_bytes in pa.h: partials, then chunk, pair count, first
    pair of each group, group of each pair) is the rule's, exactly."""
    w = make_workload(cfg, stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    need = pa.workspace_bytes(dw.cache, dw.block_table, dw.lens, w.Hq, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    dw.decode(check=True, num_partitions=0, workspace=ws)
    torch.cuda.synchronize()
    head = w.layout == "head"
    hpg, groups = (1, w.B * w.Hkv) if head else (w.Hkv, w.B)
    max_pairs = -(-2048 // hpg) + groups
    slots = max_pairs * hpg * w.G
    off = _a256(slots * w.D * 4) + _a256(slots * 2 * 4)
    plan = ws[off:off + (groups + 3) * 4].cpu().numpy().view(np.int32)
    goff = off + _a256((groups + 3) * 4)
    pages = -(-np.clip(w.lens.reshape(-1).astype(np.int64), 0, w.W * w.S) // w.S)
    chunk = _rule_chunk(pages, hpg, w.W)
    parts = -(-pages // chunk)
    first = np.concatenate([[0], np.cumsum(parts)])
    log("plan: workload %d chunk %d pairs %d (%d waves)" % (cfg, chunk, first[-1], first[-1] * hpg))
    assert plan[0] == chunk and plan[1] == first[-1]
    assert np.array_equal(plan[2:2 + groups + 1], first)
    grp = ws[goff:goff + int(first[-1]) * 4].cpu().numpy().view(np.int32)
    assert np.array_equal(grp, np.repeat(np.arange(groups), parts))
    assert first[-1] * hpg <= 2048
