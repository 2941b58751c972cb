"""Pins for the oracle's decode attention (CPU only).

P1 dense equivalence, P2 closed forms, P3 page-permutation invariance,
P4 brute force at 50 digits, P5 split/merge identity.
"""
import mpmath
import numpy as np
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload, to_bf16_bits
from oracle import (
    OracleCache,
    attention_f64,
    bf16_to_f64,
    gather_unit,
    lse_merge,
    lse_partial,
    oracle_append,
    oracle_decode,
)
from tests.oracle_fill import dense_tokens, oracle_fill


def _dense_attention(q_bits, K_bits, V_bits, sigma):
    """Non-paged textbook attention on the raw token values (the M x N matrix view)."""
    q = bf16_to_f64(q_bits)
    K, V = bf16_to_f64(K_bits), bf16_to_f64(V_bits)
    s = float(sigma) * (K @ q)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


@pytest.mark.parametrize("cfg,kw", [(1, {}), (2, dict(batch=3, lens=[1, 17, 300])),
                                    (4, dict(batch=2))])
def test_p1_paged_equals_dense(cfg, kw):
    if cfg == 4:
        kw = dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2, 3, 4, 700, 9, 31, 32, 48]]))
    w = make_workload(cfg, **kw)
    cache, kv = oracle_fill(w)
    out = oracle_decode(cache, w.q, w.block_table, w.lens, w.sigma)
    for b in range(w.B):
        for hq in range(w.Hq):
            h = hq // w.G
            K, V = dense_tokens(kv[b], w.layout, h)
            ref = _dense_attention(w.q[b, hq], K, V, w.sigma)
            assert np.max(np.abs(out[b, hq] - ref)) <= 1e-12


def _bf16(x):
    return to_bf16_bits(np.asarray(x, np.float32))


def _single_unit_cache(K_bits, V_bits, S=16, P=None, seed=0):
    """Cache holding one SEQ unit (Hkv = 1) written by oracle_append through a shuffled table."""
    L, D = K_bits.shape
    n_pages = -(-L // S)
    P = P or n_pages + 3
    rng = np.random.default_rng(seed)
    table = rng.permutation(P)[:n_pages].astype(np.int32)
    W = n_pages
    bt = np.full((1, W), 0x7FFFFFFF, np.int32)
    bt[0, :n_pages] = table
    cache = OracleCache("seq", "bf16", P, S, 1, D)
    fl = oracle_append(cache, bt, np.zeros(1, np.int32), np.array([L], np.int32),
                       K_bits[None, None], V_bits[None, None], W)
    assert fl[0] == 0
    return cache, bt


def test_p2_single_token_returns_v():
    rng = np.random.default_rng(1)
    K, V = _bf16(rng.standard_normal((1, 64))), _bf16(rng.standard_normal((1, 64)))
    cache, bt = _single_unit_cache(K, V)
    q = _bf16(rng.standard_normal((1, 1, 64)))
    out = oracle_decode(cache, q, bt, np.array([1], np.int32), np.float32(0.125))
    assert np.array_equal(out[0, 0], bf16_to_f64(V[0]))


def test_p2_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(2)
    L = 77
    K = np.repeat(_bf16(rng.standard_normal((1, 64))), L, axis=0)
    V = _bf16(rng.standard_normal((L, 64)))
    cache, bt = _single_unit_cache(K, V)
    q = _bf16(rng.standard_normal((1, 1, 64)))
    out = oracle_decode(cache, q, bt, np.array([L], np.int32), np.float32(0.125))
    assert np.max(np.abs(out[0, 0] - bf16_to_f64(V).mean(axis=0))) <= 1e-12


def test_p2_zero_query_gives_mean_and_constant_v_gives_constant():
    rng = np.random.default_rng(3)
    L = 50
    K = _bf16(rng.standard_normal((L, 64)))
    V = _bf16(rng.standard_normal((L, 64)))
    cache, bt = _single_unit_cache(K, V)
    q0 = np.zeros((1, 1, 64), np.uint16)
    out = oracle_decode(cache, q0, bt, np.array([L], np.int32), np.float32(0.125))
    assert np.max(np.abs(out[0, 0] - bf16_to_f64(V).mean(axis=0))) <= 1e-12
    c = _bf16(rng.standard_normal((1, 64)))
    Vc = np.repeat(c, L, axis=0)
    cache, bt = _single_unit_cache(K, Vc)
    q = _bf16(rng.standard_normal((1, 1, 64)))
    out = oracle_decode(cache, q, bt, np.array([L], np.int32), np.float32(0.125))
    assert np.max(np.abs(out[0, 0] - bf16_to_f64(c[0]))) <= 1e-12


def test_p2_weights_sum_to_one_and_flagged_rows_zero():
    w = make_workload(2, batch=2, lens=[40, 90])
    cache, _ = oracle_fill(w)
    K, V = gather_unit(cache, w.block_table[0], 3, 40)
    _, weights = attention_f64(bf16_to_f64(w.q[0, 12]), K, V, w.sigma)
    assert abs(weights.sum() - 1.0) <= 1e-13 and np.all(weights >= 0)
    out = oracle_decode(cache, w.q, w.block_table, w.lens, w.sigma, flags=np.array([0, 4], np.uint32))
    assert np.all(out[1] == 0) and np.any(out[0] != 0)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_p3_page_permutation_invariance(cfg):
    kw = dict(batch=2, lens=[35, 200]) if cfg != 4 else dict(
        lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2, 3, 4, 70, 9, 31, 32, 48]]))
    w = make_workload(cfg, **kw)
    cache, _ = oracle_fill(w)
    out = oracle_decode(cache, w.q, w.block_table, w.lens, w.sigma)
    perm = np.random.default_rng(11).permutation(w.P)
    c2 = cache.copy()
    c2.k = np.empty_like(cache.k); c2.k[perm] = cache.k
    c2.v = np.empty_like(cache.v); c2.v[perm] = cache.v
    if cache.k_scale is not None:
        c2.k_scale = np.empty_like(cache.k_scale); c2.k_scale[perm] = cache.k_scale
        c2.v_scale = np.empty_like(cache.v_scale); c2.v_scale[perm] = cache.v_scale
    bt2 = w.block_table.copy()
    used = bt2 != 0x7FFFFFFF
    bt2[used] = perm[bt2[used]]
    out2 = oracle_decode(c2, w.q, bt2, w.lens, w.sigma)
    assert np.array_equal(out, out2)


def _mp_attention(q, K, V, sigma):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(float(sigma)) * mpmath.fsum(mpmath.mpf(q[d]) * mpmath.mpf(K[t][d])
                                                for d in range(len(q))) for t in range(len(K))]
    m = max(s)
    e = [mpmath.exp(x - m) for x in s]
    den = mpmath.fsum(e)
    return [float(mpmath.fsum(e[t] * mpmath.mpf(V[t][d]) for t in range(len(K))) / den)
            for d in range(len(q))]


@pytest.mark.parametrize("S,L,D,Hq,Hkv", [(1, 7, 4, 2, 1), (2, 13, 8, 4, 2), (16, 40, 8, 4, 2),
                                          (16, 16, 4, 2, 2), (2, 1, 8, 4, 1)])
def test_p4_brute_force_tiny(S, L, D, Hq, Hkv):
    """Append through a shuffled table with page size S, decode, compare at 50 digits."""
    rng = np.random.default_rng(S * 1000 + L)
    B = 2
    n_pages = -(-L // S)
    P = B * n_pages + 5
    perm = rng.permutation(P).astype(np.int32)
    W = n_pages + 1
    bt = np.full((B, W), 0x7FFFFFFF, np.int32)
    for b in range(B):
        bt[b, :n_pages] = perm[b * n_pages:(b + 1) * n_pages]
    K = _bf16(rng.standard_normal((B, Hkv, L, D)) * 2)
    V = _bf16(rng.standard_normal((B, Hkv, L, D)))
    q = _bf16(rng.standard_normal((B, Hq, D)))
    cache = OracleCache("seq", "bf16", P, S, Hkv, D)
    # two appends per sequence: L-1 then 1, crossing page boundaries
    oracle_append(cache, bt, np.zeros(B, np.int32), np.full(B, L - 1, np.int32), K[:, :, :L - 1], V[:, :, :L - 1], W)
    oracle_append(cache, bt, np.full(B, L - 1, np.int32), np.ones(B, np.int32), K[:, :, L - 1:], V[:, :, L - 1:], W)
    sigma = np.float32(1 / np.sqrt(D))
    out = oracle_decode(cache, q, bt, np.full(B, L, np.int32), sigma)
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            ref = _mp_attention(bf16_to_f64(q[b, hq]).tolist(), bf16_to_f64(K[b, h]).tolist(),
                                bf16_to_f64(V[b, h]).tolist(), sigma)
            assert np.max(np.abs(out[b, hq] - np.array(ref))) <= 1e-13


def test_p5_split_merge_identity():
    rng = np.random.default_rng(9)
    L, D = 1000, 64
    K = bf16_to_f64(_bf16(rng.standard_normal((L, D)) * 3))
    V = bf16_to_f64(_bf16(rng.standard_normal((L, D))))
    q = bf16_to_f64(_bf16(rng.standard_normal(D)))
    ref, _ = attention_f64(q, K, V, 0.125)
    for n_parts in (1, 2, 7, 64):
        cuts = np.sort(rng.choice(np.arange(1, L), n_parts - 1, replace=False))
        bounds = np.concatenate([[0], cuts, [L]])
        parts = [lse_partial(q, K[a:b], V[a:b], 0.125) for a, b in zip(bounds[:-1], bounds[1:])]
        assert np.max(np.abs(lse_merge(parts) - ref)) <= 1e-12
