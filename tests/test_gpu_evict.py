"""Eviction support on the GPU against the oracle: scored decode and compaction.

Scored decode: outputs bit-identical to pa_decode at the same partition
count; every score slot a unit reads grows by the oracle's attention mass
(relative error <= 1e-4: the scores, the exp2 and the row sums are fp32,
each ~1e-6 relative, and the mass of a token is a sum of G such products);
every other slot (flagged sequences, past L, unread pages) is unchanged
bit for bit.  Compaction: pool bytes, FP8 scales and moved scores bit-exact
against the oracle; decode over the compacted cache within the decode bar.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.layout import pool_to_logical
from decode_attention_paged_pa_amd.workloads import make_workload
from oracle import oracle_compact, oracle_decode, units
from tests.oracle_fill import oracle_fill, oracle_sequences_parallel
from tests.test_gpu_parity import MAX_ABS, MEAN_ABS, flags_of, log, out_f64

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-9


def _expected_scores(w, ora, seqs, steps, base):
    """base + steps * mass at the physical slots of the sampled sequences."""
    exp = base.copy()
    for b in seqs:
        for h, m in ora[b]["mass"].items():
            row = (b,) if w.layout == "seq" else (b, h)
            ph = h if w.layout == "seq" else 0
            t = np.arange(len(m))
            pids = w.block_table[row][t // w.S]
            exp[pids, ph, t % w.S] = base[pids, ph, t % w.S] + steps * m
    return exp


def _read_slots(w, seqs):
    """Boolean mask of the score slots the units of `seqs` read."""
    ph_n = w.Hkv if w.layout == "seq" else 1
    mask = np.zeros((w.P, ph_n, w.S), bool)
    for (b, h, row, ph) in units(w.layout, w.B, w.Hkv):
        if b not in seqs:
            continue
        L = int(w.lens[row])
        t = np.arange(L)
        mask[w.block_table[row][t // w.S], ph, t % w.S] = True
    return mask


def scored_case(w, seqs, partitions, steps=1, flagged=()):
    log("scored: workload %d (%s) B=%d lens[:6]=%s" % (w.cfg_id, w.name, w.B,
                                                      w.lens.ravel()[:6].tolist()))
    dw = build_device_workload(w)
    dw.step_append()
    for b in flagged:                      # stale expected tag: the request is aborted
        dw.expected_tags[b].view(-1)[0] ^= 1
    ora = oracle_sequences_parallel(w, [b for b in seqs if b not in flagged], with_mass=True,
                                    with_pools=False)
    rng = np.random.default_rng(w.cfg_id)
    live = [b for b in seqs if b not in flagged]
    read = _read_slots(w, live)
    for p in partitions:
        plain = dw.decode(num_partitions=p).clone()
        # random prior scores (the update is a read-modify-write), except on about
        # half of the read slots, where a zero prior makes the mass itself visible
        bn = rng.random(dw.cache.new_scores().shape).astype(np.float32)
        bn[read & (rng.random(bn.shape) < 0.5)] = 0.0
        base = torch.from_numpy(bn).cuda()
        scores = base.clone()
        for _ in range(steps):
            out = pa.decode_scored(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, scores,
                                   expected_tags=dw.expected_tags, flags=dw.flags,
                                   num_partitions=p)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), plain.view(torch.int16)), "outputs differ"
        fl = flags_of(dw)
        assert all(fl[b] != 0 for b in flagged) and all(
            fl[b] == 0 for b in range(w.B) if b not in flagged)
        got = scores.cpu().numpy()
        exp = _expected_scores(w, ora, live, steps, bn)
        sampled = read
        d = got[sampled].astype(np.float64) - exp[sampled]
        inc = exp[sampled] - bn[sampled]
        rel = np.abs(d) / np.maximum(inc, 1e-30)
        log("partitions=%d steps=%d: %d slots, max rel err %.3g, max abs err %.3g" % (
            p, steps, sampled.sum(), rel.max(), np.abs(d).max()))
        assert np.all(np.abs(d) <= RTOL * inc + ATOL + 2 ** -23 * np.abs(exp[sampled]))
        untouched = ~_read_slots(w, [b for b in range(w.B) if b not in flagged])
        assert np.array_equal(got[untouched], bn[untouched])
    return dw


def test_scored_tiny_partitions():
    scored_case(make_workload(1), seqs=range(4), partitions=(0, 1, 2, 32))


def test_scored_two_steps_accumulate_and_flagged_untouched():
    w = make_workload(2, batch=4, lens=[1, 17, 300, 2000])
    scored_case(w, seqs=range(4), partitions=(0, 8), steps=2, flagged=(2,))


def test_scored_fp8():
    w = make_workload(3, batch=4, lens=[5, 700, 2049, 5000], stale_frac=0.0)
    scored_case(w, seqs=range(4), partitions=(0, 1, 4))   # 1: a 313-page run, two id segments


def test_scored_headwise():
    lens = np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2048, 8, 4096, 4097, 15, 16, 31, 1000]])
    scored_case(make_workload(4, lens=lens), seqs=range(2), partitions=(0, 1, 16, 64))


@pytest.mark.parametrize("layout,D", [("head", 128), ("head", 64), ("seq", 64)])
def test_scored_fp8_other_formats(layout, D):
    if layout == "head":
        lens = np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2048, 8, 4096, 4097, 15, 16, 31, 1000]])
    else:
        lens = [5, 700, 2049, 5000]
    w = make_workload(2, lens=lens, kv="fp8", layout=layout, head_dim=D, stale_frac=0.0)
    scored_case(w, seqs=range(w.B), partitions=(0, 4))


# ------------------------------------------------------------ compaction
def _keep_lists(w, rng, frac, reverse_unit=None):
    """Keep lists per unit ([B][Hkv][K] and the lens-shaped counts).  SEQ: one count
    per sequence, different positions per head."""
    K = int(w.lens.max())
    keep = np.zeros((w.B, w.Hkv, max(K, 1)), np.int32)
    if w.layout == "seq":
        n_keep = np.array([max(1, int(round(int(L) * frac))) for L in w.lens], np.int32)
    else:
        n_keep = np.maximum(1, np.round(w.lens * frac)).astype(np.int32)
    for (b, h, row, _) in units(w.layout, w.B, w.Hkv):
        L, n = int(w.lens[row]), int(n_keep[row])
        pos = np.sort(rng.choice(L, n, replace=False))
        if reverse_unit == (b, h):
            pos = pos[::-1]
        keep[b, h, :n] = pos
    return keep, n_keep


def _new_table(w, n_keep):
    used = set(w.block_table[w.block_table != 0x7FFFFFFF].tolist())
    free = [p for p in range(w.P) if p not in used]
    nt = np.full(w.block_table.shape, 0x7FFFFFFF, np.int32)
    k = 0
    rows = [(b,) for b in range(w.B)] if w.layout == "seq" else [
        (b, h) for b in range(w.B) for h in range(w.Hkv)]
    for row in rows:
        need = -(-int(n_keep[row]) // w.S)
        assert k + need <= len(free), "not enough spare pages"
        nt[row][:need] = free[k:k + need]
        k += need
    return nt


def _unit_arrays(w, keep, n_keep):
    """The oracle's per-unit view of the keep lists."""
    ks, ns = [], []
    for (b, h, row, _) in units(w.layout, w.B, w.Hkv):
        ks.append(keep[b, h]); ns.append(int(n_keep[row]))
    return np.stack(ks), np.array(ns, np.int32)


@pytest.mark.parametrize("cfg,kw,frac", [
    (2, dict(batch=3, lens=[5, 100, 700], spare_pages=64), 0.3),
    (3, dict(batch=3, lens=[40, 333, 1500], spare_pages=96, stale_frac=0.0), 0.25),
    (4, dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2048, 8, 4096, 4097, 15, 16, 31, 1000]]),
             spare_pages=700), 0.125),
    (1, dict(spare_pages=64), 0.5),
    (2, dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64], [300, 8, 1000, 4097, 15, 16, 31, 90]]),
             kv="fp8", layout="head", head_dim=64, spare_pages=200), 0.25),
    (2, dict(batch=3, lens=[40, 333, 1500], kv="fp8", head_dim=64, spare_pages=96), 0.5),
])
def test_compaction_matches_oracle(cfg, kw, frac):
    w = make_workload(cfg, **kw)
    log("compact: workload %d (%s) layout=%s kv=%s P=%d keep %.3f" % (
        w.cfg_id, w.name, w.layout, w.kv_dtype, w.P, frac))
    dw = build_device_workload(w)
    dw.step_append()
    cache_o, _ = oracle_fill(w)
    rng = np.random.default_rng(cfg)
    keep, n_keep = _keep_lists(w, rng, frac, reverse_unit=(0, 1))
    nt = _new_table(w, n_keep)
    scores0 = rng.random(dw.cache.new_scores().shape).astype(np.float32)
    scores = torch.from_numpy(scores0).cuda()
    keep_d = torch.from_numpy(keep).cuda()
    n_keep_d = torch.from_numpy(n_keep).cuda()
    nt_d = torch.from_numpy(nt).cuda()
    pa.compact(dw.cache, dw.block_table, dw.lens, keep_d, n_keep_d, nt_d, scores=scores,
               flags=dw.flags)
    torch.cuda.synchronize()
    assert np.all(flags_of(dw) == 0)
    ku, nu = _unit_arrays(w, keep, n_keep)
    c2, s2 = oracle_compact(cache_o, w.block_table, w.lens, ku, nu, nt, scores=scores0)
    new_pages = np.unique(nt[nt != 0x7FFFFFFF])
    for which in ("k", "v"):
        raw = (dw.cache.k if which == "k" else dw.cache.v).cpu().numpy()
        logical = pool_to_logical(raw, which, w.layout, w.kv_dtype, w.P, w.Hkv, w.D)
        want = (c2.k if which == "k" else c2.v)
        bad = np.argwhere(logical[new_pages] != want[new_pages])
        assert bad.size == 0, "%s differs at %d places, first %s" % (which, len(bad), bad[:3].tolist())
    if w.kv_dtype == "fp8":
        for mine, theirs in ((dw.cache.k_scale, c2.k_scale), (dw.cache.v_scale, c2.v_scale)):
            assert np.array_equal(mine.cpu().numpy()[new_pages].view(np.uint32),
                                  theirs[new_pages].view(np.uint32))
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), s2.view(np.uint32))
    # decode over the compacted cache, lengths n_keep
    out = pa.decode(dw.cache, dw.q, nt_d, n_keep_d, w.sigma, num_partitions=0)
    torch.cuda.synchronize()
    ref = oracle_decode(c2, w.q, nt, n_keep, w.sigma)
    e = np.abs(out_f64(out) - ref)
    log("decode after compaction: max-abs %.3g mean-abs %.3g" % (e.max(), e.mean()))
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_compaction_flags_and_skipped_tokens():
    w = make_workload(2, batch=3, lens=[40, 100, 70], spare_pages=32)
    dw = build_device_workload(w)
    dw.step_append()
    keep, n_keep = _keep_lists(w, np.random.default_rng(3), 0.5)
    keep[1, 2, 3] = 100                    # == len: outside [0, len)
    nt = _new_table(w, n_keep)
    nt[2, 1] = w.P + 5                     # a destination page outside the pool
    before = dw.cache.k.clone()
    pa.compact(dw.cache, dw.block_table, dw.lens, torch.from_numpy(keep).cuda(),
               torch.from_numpy(n_keep).cuda(), torch.from_numpy(nt).cuda(), flags=dw.flags)
    torch.cuda.synchronize()
    assert flags_of(dw).tolist() == [0, 8, 2]
    # pages of the old table are never written
    old = np.unique(w.block_table[w.block_table != 0x7FFFFFFF])
    raw0 = pool_to_logical(before.cpu().numpy(), "k", w.layout, w.kv_dtype, w.P, w.Hkv, w.D)
    raw1 = pool_to_logical(dw.cache.k.cpu().numpy(), "k", w.layout, w.kv_dtype, w.P, w.Hkv, w.D)
    assert np.array_equal(raw0[old], raw1[old])


def test_score_then_compact_then_decode():
    """The eviction loop: scored steps, keep the top-scored eighth or quarter per
    head (HEAD layout: heads keep different counts), compact, decode again.  The
    keep lists come from the oracle's masses; the GPU's own top sets must agree
    with them almost everywhere."""
    from oracle import oracle_attention_mass

    lens = np.array([[600, 1000, 333, 2048, 64, 128, 900, 40]])
    w = make_workload(4, lens=lens, spare_pages=200)
    dw = build_device_workload(w)
    dw.step_append()
    scores = dw.cache.new_scores()
    for _ in range(2):
        pa.decode_scored(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, scores)
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    cache_o, _ = oracle_fill(w)
    mass = oracle_attention_mass(cache_o, w.q, w.block_table, w.lens, w.sigma)
    keep = np.zeros((1, w.Hkv, int(lens.max())), np.int32)
    n_keep = np.zeros((1, w.Hkv), np.int32)
    agree = total = 0
    for h in range(w.Hkv):
        L = int(lens[0, h])
        n = max(1, L // 8 if h % 2 == 0 else L // 4)          # per-head rates
        top = np.sort(np.argsort(-mass[(0, h)], kind="stable")[:n])
        keep[0, h, :n] = top
        n_keep[0, h] = n
        t = np.arange(L)
        mine = np.argsort(-sc[w.block_table[0, h][t // w.S], 0, t % w.S], kind="stable")[:n]
        agree += len(set(mine.tolist()) & set(top.tolist()))
        total += n
    log("top-score sets: GPU and oracle agree on %d of %d kept tokens" % (agree, total))
    assert agree >= 0.99 * total
    nt = _new_table(w, n_keep)
    nt_d, n_keep_d = torch.from_numpy(nt).cuda(), torch.from_numpy(n_keep).cuda()
    pa.compact(dw.cache, dw.block_table, dw.lens, torch.from_numpy(keep).cuda(), n_keep_d, nt_d,
               scores=scores)
    out = pa.decode(dw.cache, dw.q, nt_d, n_keep_d, w.sigma)
    torch.cuda.synchronize()
    ku, nu = _unit_arrays(w, keep, n_keep)
    c2, _ = oracle_compact(cache_o, w.block_table, w.lens, ku, nu, nt)
    ref = oracle_decode(c2, w.q, nt, n_keep, w.sigma)
    e = np.abs(out_f64(out) - ref)
    log("evict loop: max-abs %.3g" % e.max())
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS
