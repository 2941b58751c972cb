"""Pins for the oracle's append (FP8 quantisation) and tag validation (CPU only).

P8: after random append sequences the per-(page, head) scale equals
fl32(amax / 448) over the values written since the page was fresh, the
largest of them encodes to +-448, and every value decodes back within the
e4m3 error bound.  P9: flags built by construction (stale tags, out-of-range
ids, oversize lengths) are reproduced exactly.
"""
import numpy as np
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload, to_bf16_bits
from oracle import (
    FLAG_LEN_OVERFLOW,
    FLAG_PAGE_OOB,
    FLAG_TAG_MISMATCH,
    OracleCache,
    bf16_to_f64,
    e4m3_to_f64,
    oracle_append,
    oracle_validate,
)
from tests.oracle_fill import oracle_fill


def _random_append_run(seed, layout):
    rng = np.random.default_rng(seed)
    B, Hkv, D, S = 3, 2, 16, 16
    W = 6
    P = B * W * (Hkv if layout == "head" else 1) + 4
    perm = rng.permutation(P).astype(np.int32)
    shape = (B, W) if layout == "seq" else (B, Hkv, W)
    bt = perm[:int(np.prod(shape))].reshape(shape)
    lshape = (B,) if layout == "seq" else (B, Hkv)
    cache = OracleCache(layout, "fp8", P, S, Hkv, D)
    lens = np.zeros(lshape, np.int32)
    # independent record: for each (page, head, K/V) the fp32 values written since fresh,
    # and for each written slot the original value and how many times it was quantised
    hist = {}
    orig = {}
    for step in range(12):
        n = rng.integers(0, 23, size=lshape).astype(np.int32)
        n = np.minimum(n, W * S - lens)
        n_max = int(n.max()) if n.size else 0
        scale = np.exp(rng.uniform(-3, 3))
        kx = rng.standard_normal((B, Hkv, max(n_max, 1), D)).astype(np.float32) * scale
        vx = rng.standard_normal((B, Hkv, max(n_max, 1), D)).astype(np.float32) * scale * 0.5
        kb, vb = to_bf16_bits(kx), to_bf16_bits(vx)
        fl = oracle_append(cache, bt, lens, n, kb, vb, W)
        assert np.all(fl == 0)
        for b in range(B):
            for h in range(Hkv):
                row = (b,) if layout == "seq" else (b, h)
                ph = h if layout == "seq" else 0
                for t in range(int(n[row])):
                    pos = int(lens[row]) + t
                    pid = int(bt[row][pos // S])
                    slot = pos % S
                    for kv, src in (("k", kb), ("v", vb)):
                        key = (pid, ph, kv)
                        # a page is fresh when this call's first write to it lands on slot 0
                        first_pos_in_call = max(int(lens[row]), (pos // S) * S)
                        if first_pos_in_call % S == 0 and pos == first_pos_in_call:
                            hist[key] = []
                            for s2 in range(S):
                                orig.pop((pid, ph, s2, kv), None)
                        hist[key].append(bf16_to_f64(src[b, h, t]))
                        for s2 in range(S):
                            if (pid, ph, s2, kv) in orig:
                                orig[(pid, ph, s2, kv)][1] += 1
                        orig[(pid, ph, slot, kv)] = [bf16_to_f64(src[b, h, t]), 0]
        lens = lens + n
    return cache, hist, orig


@pytest.mark.parametrize("layout", ["seq", "head"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_p8_scale_invariant_and_error_bound(layout, seed):
    cache, hist, orig = _random_append_run(seed, layout)
    for (pid, ph, kv), vals in hist.items():
        scales = cache.k_scale if kv == "k" else cache.v_scale
        amax = np.float32(np.max(np.abs(np.concatenate(vals))))
        assert scales[pid, ph] == np.float32(amax / np.float32(448.0)), (pid, ph, kv)
        pool = cache.k if kv == "k" else cache.v
        n_written = sum(1 for (p, hh, s, k2) in orig if (p, hh, k2) == (pid, ph, kv))
        codes = pool[pid, ph, :n_written]
        assert np.max(np.abs(e4m3_to_f64(codes))) == 448.0
    for (pid, ph, slot, kv), (x, n_requant) in orig.items():
        scales = cache.k_scale if kv == "k" else cache.v_scale
        pool = cache.k if kv == "k" else cache.v
        s = float(scales[pid, ph])
        got = e4m3_to_f64(pool[pid, ph, slot]) * s
        n_q = 1 + n_requant   # an upper bound on the number of roundings it went through
        bound = n_q * (np.abs(x) * 2.0 ** -4 * 1.07 + s * 2.0 ** -10 * 1.01)
        assert np.all(np.abs(got - x) <= bound + 1e-30), (pid, ph, slot, kv)


def test_bf16_append_is_a_copy_and_leaves_other_slots():
    w = make_workload(2, batch=2, lens=[20, 33])
    cache, kv = oracle_fill(w)
    k_hist, v_hist, k_new, _, n_hist = kv[1]
    pid0, pid2 = w.block_table[1, 0], w.block_table[1, 2]
    assert np.array_equal(cache.k[pid0, 5, :16], k_hist[5, :16])
    assert np.array_equal(cache.k[pid2, 5, 0], k_new[5, 0])          # token 32 = the new one
    assert np.all(cache.k[pid2, 5, 1:] == 0x7FC0)                    # untouched poison


def test_append_flags_oob_and_overflow():
    cache = OracleCache("seq", "bf16", 8, 16, 1, 4)
    bt = np.array([[0, 1], [2, 99], [3, 4]], np.int32)
    kb = np.zeros((3, 1, 40, 4), np.uint16)
    fl = oracle_append(cache, bt, np.array([0, 0, 0], np.int32), np.array([10, 20, 33], np.int32), kb, kb, 2)
    assert fl.tolist() == [0, FLAG_PAGE_OOB, FLAG_LEN_OVERFLOW]
    assert np.all(cache.k[4, 0] == 0)        # in-range part of the overflowing append is written


def test_p9_stale_tags_flag_exactly_the_affected_sequences():
    w = make_workload(3, batch=8, lens=[400, 1000, 16, 17, 300, 5000, 64, 1], stale_frac=0.05)
    fl = oracle_validate(w.layout, w.P, w.S, w.block_table, w.lens, w.page_tags, w.expected_tags, w.W)
    expect = np.array([FLAG_TAG_MISMATCH if w.stale[b].any() else 0 for b in range(w.B)], np.uint32)
    assert w.stale.any() and not w.stale.all()
    assert np.array_equal(fl, expect)
    # no-op tracker: no tag compare at all
    fl0 = oracle_validate(w.layout, w.P, w.S, w.block_table, w.lens, w.page_tags, None, w.W)
    assert np.all(fl0 == 0)


def test_p9_headwise_flags_or_over_heads_and_brute_force():
    lens = np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2, 3, 4, 70, 9, 31, 32, 48],
                     [0, 0, 0, 0, 0, 0, 0, 0]])
    w = make_workload(4, lens=lens, table_width=40, stale_frac=0.0)
    exp = w.expected_tags.copy()
    bt = w.block_table.copy()
    L = w.lens.copy()
    exp[0, 6, 0] ^= 1          # stale in sequence 0, head 6
    bt[1, 3, 4] = w.P + 5      # out of range in sequence 1, head 3
    L[2, 1] = 40 * 16 + 1      # too long in sequence 2
    bt[2, 1, :] = 0
    exp[2, 1, :] = w.page_tags[0]
    fl = oracle_validate(w.layout, w.P, w.S, bt, L, w.page_tags, exp, 40)
    assert fl.tolist() == [FLAG_TAG_MISMATCH, FLAG_PAGE_OOB, FLAG_LEN_OVERFLOW]
    # brute force over every (b, h, i) with the rule written as a predicate
    bf = np.zeros(3, np.uint32)
    for b in range(3):
        for h in range(8):
            n = -(-min(int(L[b, h]), 640) // 16)
            if L[b, h] > 640:
                bf[b] |= 4
            for i in range(n):
                p = int(bt[b, h, i])
                bf[b] |= 2 if not 0 <= p < w.P else (1 if exp[b, h, i] != w.page_tags[p] else 0)
    assert np.array_equal(bf, fl)


def test_p9_unread_entries_are_not_checked():
    w = make_workload(2, batch=2, lens=[16, 17], stale_frac=0.0)
    exp = w.expected_tags.copy()
    bt = w.block_table.copy()
    exp[0, 1] ^= 7             # entry 1 of a 16-token sequence is never read
    bt[0, 2] = -5
    fl = oracle_validate(w.layout, w.P, w.S, bt, w.lens, w.page_tags, exp, w.W)
    assert fl.tolist() == [0, 0]


def _gated_case(kv):
    """Two SEQ sequences; sequence 1's entry 2 is stale and names page 5, which
    belongs to sequence 0 now (sequence 0 writes into it in the same call)."""
    S, D, W, P = 16, 4, 4, 12
    bt = np.array([[4, 5, 9, 10], [0, 1, 5, 11]], np.int32)
    tags = np.arange(100, 100 + P, dtype=np.uint32)
    exp = tags[np.clip(bt, 0, P - 1)].astype(np.uint32)
    exp[1, 2] = tags[5] - 1                       # the tag page 5 had before reallocation
    lens_old = np.array([20, 30], np.int32)       # seq 0 writes pages 5 and 9; seq 1 pages 1 and 5
    n_new = np.array([14, 5], np.int32)
    rng = np.random.default_rng(3)
    k = to_bf16_bits(rng.standard_normal((2, 1, 14, D)).astype(np.float32))
    v = to_bf16_bits(rng.standard_normal((2, 1, 14, D)).astype(np.float32))
    cache = OracleCache("seq", kv, P, S, 1, D)
    fl = oracle_append(cache, bt, lens_old, n_new, k, v, W, expected_tags=exp, page_tags=tags)
    return cache, fl, bt, exp, tags, lens_old, n_new, k, v


def test_p10_append_skips_pages_whose_tag_is_stale():
    """R5's gate: sequence 1's two tokens for page 5 (through its stale entry) are
    not written and flag bit 0; everything else is written; brute force over
    every token with the rule written as a predicate."""
    cache, fl, bt, exp, tags, lens_old, n_new, k, v = _gated_case("bf16")
    assert fl.tolist() == [0, FLAG_TAG_MISMATCH]
    want_k = np.full(cache.k.shape, 0x7FC0, np.uint16)
    for b in range(2):
        for t in range(int(n_new[b])):
            pos = int(lens_old[b]) + t
            i, slot = pos // 16, pos % 16
            pid = int(bt[b, i])
            if exp[b, i] == tags[pid]:
                want_k[pid, 0, slot] = k[b, 0, t]
    assert np.array_equal(cache.k, want_k)
    assert np.all(cache.k[5, 0, :4] == 0x7FC0)                 # seq 0 starts page 5 at slot 4
    assert np.array_equal(cache.k[5, 0, 4:16], k[0, 0, :12])   # seq 0's tokens, not seq 1's


def test_p10_fp8_page_behind_a_stale_entry_keeps_codes_and_scale():
    cache, fl, bt, exp, tags, lens_old, n_new, k, v = _gated_case("fp8")
    assert fl.tolist() == [0, FLAG_TAG_MISMATCH]
    # pages 5 and 9 are exactly what sequence 0's append alone makes of them
    only0 = OracleCache("seq", "fp8", 12, 16, 1, 4)
    oracle_append(only0, bt, lens_old, np.array([14, 0], np.int32), k, v, 4,
                  expected_tags=exp, page_tags=tags)
    for p in (5, 9):
        assert np.array_equal(cache.k[p], only0.k[p]) and np.array_equal(cache.v[p], only0.v[p])
        assert cache.k_scale[p, 0].tobytes() == only0.k_scale[p, 0].tobytes()
        assert cache.v_scale[p, 0].tobytes() == only0.v_scale[p, 0].tobytes()


def test_p10_no_expected_tags_no_gate():
    """Without expected tags the append checks none (sequence 1 overwrites slots
    of page 5: the hazard the gate removes)."""
    _, _, bt, exp, tags, lens_old, n_new, k, v = _gated_case("bf16")
    cache = OracleCache("seq", "bf16", 12, 16, 1, 4)
    fl = oracle_append(cache, bt, lens_old, n_new, k, v, 4)
    assert fl.tolist() == [0, 0]
    assert np.array_equal(cache.k[5, 0, 0:3], k[1, 0, 2:5])    # positions 32..34 of seq 1
