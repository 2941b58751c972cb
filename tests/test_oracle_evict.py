"""Pins for the oracle's eviction support: attention-mass scores and compaction (CPU).

E1 conservation: each query head's weights sum to 1, so a unit's masses sum
to G; E2 closed forms (identical keys -> G / L each; one dominant key);
E3 50-digit brute force on tiny paged shapes; E4 the paged score update
touches exactly the slots it should and conserves the added mass, invariant
under page renumbering; E5 compaction of BF16 is a gather (dense identity,
attention on the compacted cache equals attention on the kept tokens);
E6 compaction of FP8 keeps the scale invariant and the e4m3 error bound,
and a full-page identity keep round-trips the codes; E7 scores move with
their tokens.
"""
import mpmath
import numpy as np
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload, to_bf16_bits
from oracle import (
    E4M3_MAX,
    OracleCache,
    bf16_to_f64,
    e4m3_to_f64,
    gather_unit,
    oracle_append,
    oracle_attention_mass,
    oracle_compact,
    oracle_decode,
    oracle_score_update,
    units,
)
from tests.oracle_fill import dense_tokens, oracle_fill


def _bf16(x):
    return to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("cfg,kw", [(1, {}), (3, dict(batch=2, lens=[20, 300])),
                                    (4, dict(batch=1))])
def test_e1_mass_sums_to_group_size(cfg, kw):
    if cfg == 4:
        kw = dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64]]))
    w = make_workload(cfg, **kw)
    cache, _ = oracle_fill(w)
    mass = oracle_attention_mass(cache, w.q, w.block_table, w.lens, w.sigma)
    assert len(mass) == w.B * w.Hkv
    for (b, h), m in mass.items():
        L = int(w.lens[b] if w.layout == "seq" else w.lens[b, h])
        assert m.shape == (L,) and np.all(m >= 0)
        assert abs(m.sum() - w.G) <= 1e-12 * w.G


def _unit(K_bits, V_bits, S=16, seed=0, kv="bf16"):
    L, D = K_bits.shape
    n_pages = -(-L // S)
    P = n_pages + 3
    rng = np.random.default_rng(seed)
    bt = np.full((1, n_pages + 1), 0x7FFFFFFF, np.int32)
    bt[0, :n_pages] = rng.permutation(P)[:n_pages]
    cache = OracleCache("seq", kv, P, S, 1, D)
    fl = oracle_append(cache, bt, np.zeros(1, np.int32), np.array([L], np.int32),
                       K_bits[None, None], V_bits[None, None], n_pages + 1)
    assert fl[0] == 0
    return cache, bt


def test_e2_identical_keys_spread_mass_evenly():
    rng = np.random.default_rng(3)
    L, G = 77, 4
    K = np.repeat(_bf16(rng.standard_normal((1, 64))), L, axis=0)
    V = _bf16(rng.standard_normal((L, 64)))
    cache, bt = _unit(K, V)
    q = _bf16(rng.standard_normal((1, G, 64)))
    m = oracle_attention_mass(cache, q, bt, np.array([L], np.int32), np.float32(0.125))[(0, 0)]
    assert np.max(np.abs(m - G / L)) <= 1e-14


def test_e2_dominant_key():
    """Every head's query is aligned with key j (score 8 nats above the rest)."""
    L, G, D = 40, 3, 64
    qv = np.zeros(D, np.float32); qv[5] = 1.0
    K = np.zeros((L, D), np.float32); K[17, 5] = 64.0
    V = np.random.default_rng(4).standard_normal((L, D)).astype(np.float32)
    cache, bt = _unit(_bf16(K), _bf16(V))
    q = np.repeat(_bf16(qv)[None, None], G, axis=1)
    m = oracle_attention_mass(cache, q, bt, np.array([L], np.int32), np.float32(0.125))[(0, 0)]
    wj = np.exp(8.0) / (np.exp(8.0) + L - 1)
    assert abs(m[17] - G * wj) <= 1e-12
    others = np.delete(m, 17)
    assert np.max(np.abs(others - G * (1 - wj) / (L - 1))) <= 1e-14


def _mp_weights(q, K, sigma):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(float(sigma)) * mpmath.fsum(mpmath.mpf(q[d]) * mpmath.mpf(K[t][d])
                                                for d in range(len(q))) for t in range(len(K))]
    mx = max(s)
    e = [mpmath.exp(x - mx) for x in s]
    den = mpmath.fsum(e)
    return [float(x / den) for x in e]


@pytest.mark.parametrize("S,L,D,Hq,Hkv", [(2, 9, 4, 4, 2), (16, 20, 8, 4, 1), (4, 13, 4, 6, 3)])
def test_e3_brute_force_tiny(S, L, D, Hq, Hkv):
    rng = np.random.default_rng(S * 100 + L)
    B = 2
    n_pages = -(-L // S)
    P = B * n_pages + 2
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((B, n_pages + 1), 0x7FFFFFFF, np.int32)
    for b in range(B):
        bt[b, :n_pages] = perm[b * n_pages:(b + 1) * n_pages]
    K = _bf16(rng.standard_normal((B, Hkv, L, D)) * 2)
    V = _bf16(rng.standard_normal((B, Hkv, L, D)))
    q = _bf16(rng.standard_normal((B, Hq, D)))
    cache = OracleCache("seq", "bf16", P, S, Hkv, D)
    oracle_append(cache, bt, np.zeros(B, np.int32), np.full(B, L, np.int32), K, V, n_pages + 1)
    sigma = np.float32(1 / np.sqrt(D))
    mass = oracle_attention_mass(cache, q, bt, np.full(B, L, np.int32), sigma)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            ref = np.zeros(L)
            for g in range(G):
                ref += np.array(_mp_weights(bf16_to_f64(q[b, h * G + g]).tolist(),
                                            bf16_to_f64(K[b, h]).tolist(), sigma))
            assert np.max(np.abs(mass[(b, h)] - ref)) <= 1e-14


@pytest.mark.parametrize("cfg", [2, 4])
def test_e4_score_update_touches_exactly_the_read_slots(cfg):
    kw = dict(batch=3, lens=[1, 40, 300]) if cfg == 2 else dict(
        lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2, 3, 4, 70, 9, 31, 32, 48]]))
    w = make_workload(cfg, **kw)
    cache, _ = oracle_fill(w)
    flags = np.zeros(w.B, np.uint32); flags[-1] = 1
    mass = oracle_attention_mass(cache, w.q, w.block_table, w.lens, w.sigma, flags=flags)
    ph = w.Hkv if w.layout == "seq" else 1
    base = np.random.default_rng(0).random((w.P, ph, w.S)).astype(np.float32)
    sc = oracle_score_update(w.layout, base.copy(), w.block_table, w.lens, mass, w.S)
    touched = np.zeros(sc.shape, bool)
    for (b, h, row, p_h) in units(w.layout, w.B, w.Hkv):
        if flags[b]:
            continue
        L = int(w.lens[row])
        for t in range(L):
            touched[int(w.block_table[row][t // w.S]), p_h, t % w.S] = True
    assert np.array_equal(sc[~touched], base[~touched])     # unread, past-L, flagged: untouched
    assert np.all(sc[touched] > base[touched])
    added = (sc.astype(np.float64) - base).sum()
    assert abs(added - w.G * len(mass)) <= 1e-5 * w.G * len(mass)
    # renumbering the physical pages permutes the scores the same way
    perm = np.random.default_rng(5).permutation(w.P)
    c2 = cache.copy()
    c2.k = np.empty_like(cache.k); c2.k[perm] = cache.k
    c2.v = np.empty_like(cache.v); c2.v[perm] = cache.v
    bt2 = w.block_table.copy()
    used = bt2 != 0x7FFFFFFF
    bt2[used] = perm[bt2[used]]
    mass2 = oracle_attention_mass(c2, w.q, bt2, w.lens, w.sigma, flags=flags)
    base2 = np.empty_like(base); base2[perm] = base
    sc2 = oracle_score_update(w.layout, base2, bt2, w.lens, mass2, w.S)
    assert np.array_equal(sc2[perm], sc)


def _keep_lists(w, rng, frac):
    keeps, ns = [], []
    for (b, h, row, _) in units(w.layout, w.B, w.Hkv):
        L = int(w.lens[row])
        n = max(1, int(round(L * frac))) if L else 0
        keeps.append(np.sort(rng.choice(L, n, replace=False)) if n else np.zeros(0, np.int64))
        ns.append(n)
    mk = max(ns + [1])
    keep = np.zeros((len(ns), mk), np.int32)
    for i, k in enumerate(keeps):
        keep[i, :len(k)] = k
    return keep, np.array(ns, np.int32)


def _new_table(w, n_keep, first_free):
    """Fresh pages after the pool's used ones, dealt in unit order (SEQ: a sequence's
    heads share its table row, so the row must cover the largest keep count)."""
    nt = np.full(w.block_table.shape, 0x7FFFFFFF, np.int32)
    nxt = first_free
    if w.layout == "seq":
        per_b = n_keep.reshape(w.B, w.Hkv).max(axis=1)
        for b in range(w.B):
            k = -(-int(per_b[b]) // w.S)
            nt[b, :k] = np.arange(nxt, nxt + k); nxt += k
    else:
        for b in range(w.B):
            for h in range(w.Hkv):
                k = -(-int(n_keep[b * w.Hkv + h]) // w.S)
                nt[b, h, :k] = np.arange(nxt, nxt + k); nxt += k
    return nt, nxt


def _grown(cache, extra):
    c = OracleCache(cache.layout, cache.kv_dtype, cache.P + extra, cache.S, cache.Hkv, cache.D)
    c.k[:cache.P], c.v[:cache.P] = cache.k, cache.v
    if cache.k_scale is not None:
        c.k_scale[:cache.P], c.v_scale[:cache.P] = cache.k_scale, cache.v_scale
    return c


@pytest.mark.parametrize("cfg,kw", [(2, dict(batch=3, lens=[5, 100, 700])),
                                    (4, dict(batch=1))])
def test_e5_bf16_compaction_is_a_gather(cfg, kw):
    if cfg == 4:
        kw = dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64]]))
    w = make_workload(cfg, **kw)
    cache, kv = oracle_fill(w)
    cache = _grown(cache, 200)
    rng = np.random.default_rng(7)
    keep, n_keep = _keep_lists(w, rng, 0.3)
    nt, _ = _new_table(w, n_keep, w.P)
    c2, _ = oracle_compact(cache, w.block_table, w.lens, keep, n_keep, nt)
    out2 = None
    for i, (b, h, row, ph) in enumerate(units(w.layout, w.B, w.Hkv)):
        n = int(n_keep[i])
        K, V = dense_tokens(kv[b], w.layout, h)
        Kc, Vc = gather_unit(c2, nt[row], ph, n)
        assert np.array_equal(Kc, bf16_to_f64(K[keep[i, :n]]))
        assert np.array_equal(Vc, bf16_to_f64(V[keep[i, :n]]))
    # attention over the compacted cache = attention over the kept tokens (HEAD: per-head lengths)
    if w.layout == "head":
        new_lens = n_keep.reshape(w.B, w.Hkv)
        out2 = oracle_decode(c2, w.q, nt, new_lens, w.sigma)
        for i, (b, h, row, ph) in enumerate(units(w.layout, w.B, w.Hkv)):
            K, V = dense_tokens(kv[b], w.layout, h)
            Ks, Vs = bf16_to_f64(K[keep[i, :n_keep[i]]]), bf16_to_f64(V[keep[i, :n_keep[i]]])
            for g in range(w.G):
                qq = bf16_to_f64(w.q[b, h * w.G + g])
                z = float(w.sigma) * (Ks @ qq)
                p = np.exp(z - z.max())
                assert np.max(np.abs(out2[b, h * w.G + g] - (p / p.sum()) @ Vs)) <= 1e-12


def test_e6_fp8_compaction_scale_invariant_and_error_bound():
    w = make_workload(3, batch=2, lens=[300, 1000], stale_frac=0.0)
    cache, _ = oracle_fill(w)
    cache = _grown(cache, 200)
    keep, n_keep = _keep_lists(w, np.random.default_rng(9), 0.4)
    nt, _ = _new_table(w, n_keep, w.P)
    c2, _ = oracle_compact(cache, w.block_table, w.lens, keep, n_keep, nt)
    for i, (b, h, row, ph) in enumerate(units(w.layout, w.B, w.Hkv)):
        n = int(n_keep[i])
        old_k, old_v = gather_unit(cache, w.block_table[row], ph, int(w.lens[row]))
        new_k, new_v = gather_unit(c2, nt[row], ph, n)
        for old, new, sc_new in ((old_k, new_k, c2.k_scale), (old_v, new_v, c2.v_scale)):
            x = old[keep[i, :n]]                          # the decoded old values (exact in fp32)
            for p0 in range(0, n, w.S):
                pid = int(nt[row][p0 // w.S])
                xs = x[p0:p0 + w.S]
                s = sc_new[pid, ph]
                assert s == np.float32(np.float32(np.max(np.abs(xs))) / np.float32(448))
                # e4m3 RNE: relative error <= 2^-4 for normals, absolute <= 2^-10 * s below 2^-6
                err = np.abs(new[p0:p0 + w.S] - xs)
                assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6))
                # the largest value of the page becomes the +-448 code
                j = np.unravel_index(np.argmax(np.abs(xs)), xs.shape)
                assert abs(new[p0:p0 + w.S][j]) == pytest.approx(E4M3_MAX * float(s), rel=1e-7)


def test_e6_fp8_identity_keep_round_trips_codes():
    """Keeping every token into fresh pages: codes come back equal wherever the scale does."""
    w = make_workload(3, batch=1, lens=[160], stale_frac=0.0)
    cache, _ = oracle_fill(w)
    cache = _grown(cache, 64)
    n = 160
    keep = np.tile(np.arange(n, dtype=np.int32), (w.Hkv, 1))
    n_keep = np.full(w.Hkv, n, np.int32)
    nt, _ = _new_table(w, n_keep, w.P)
    c2, _ = oracle_compact(cache, w.block_table, w.lens, keep, n_keep, nt)
    same = 0
    for i in range(10):
        po, pn = int(w.block_table[0, i]), int(nt[0, i])
        for h in range(w.Hkv):
            for pool_o, pool_n, so, sn in ((cache.k, c2.k, cache.k_scale, c2.k_scale),
                                           (cache.v, c2.v, cache.v_scale, c2.v_scale)):
                if so[po, h] == sn[pn, h]:
                    assert np.array_equal(pool_o[po, h], pool_n[pn, h])
                    same += 1
                else:   # one ulp of scale apart at most
                    assert abs(np.float64(sn[pn, h]) / so[po, h] - 1) <= 2.0 ** -22
                    assert np.max(np.abs(e4m3_to_f64(pool_o[po, h]) - e4m3_to_f64(pool_n[pn, h]))
                                  ) <= 32.0
    assert same > 0


def test_e7_scores_move_with_their_tokens():
    w = make_workload(4, lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64]]))
    cache, _ = oracle_fill(w)
    cache = _grown(cache, 100)
    scores = np.random.default_rng(1).random((cache.P, 1, w.S)).astype(np.float32)
    keep, n_keep = _keep_lists(w, np.random.default_rng(2), 0.5)
    nt, _ = _new_table(w, n_keep, w.P)
    _, s2 = oracle_compact(cache, w.block_table, w.lens, keep, n_keep, nt, scores=scores)
    for i, (b, h, row, ph) in enumerate(units(w.layout, w.B, w.Hkv)):
        for j in range(int(n_keep[i])):
            t = int(keep[i, j])
            assert s2[nt[row][j // w.S], ph, j % w.S] == scores[w.block_table[row][t // w.S], ph, t % w.S]
    # pages the new table does not name keep their old scores
    named = set(nt[nt != 0x7FFFFFFF].tolist())
    for p in range(cache.P):
        if p not in named:
            assert np.array_equal(s2[p], scores[p])
