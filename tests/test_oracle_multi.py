"""Pins for the oracle's multi-query (speculative verification) decode, CPU only.

M1 one draft is plain decode; M2 closed forms that pin the causal limit of
every draft (identical keys -> mean of V over the visible prefix; one
dominant key -> its value, only once it is visible); M3 causality invariants;
M4 brute force at 50 digits on tiny paged shapes; M5 torch's own masked
attention (CPU, fp64) on the dense tokens; M6 degenerate lengths.
"""
import mpmath
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd.workloads import make_workload, to_bf16_bits
from oracle import (
    OracleCache,
    bf16_to_f64,
    oracle_append,
    oracle_decode,
    oracle_decode_multi,
)
from tests.oracle_fill import dense_tokens, oracle_fill


def _bf16(x):
    return to_bf16_bits(np.asarray(x, np.float32))


def _unit_cache(K_bits, V_bits, T, S=16, seed=0, kv="bf16"):
    """One SEQ unit (Hkv = 1): L - T history tokens, then T drafts, via a shuffled table."""
    L, D = K_bits.shape
    n_pages = -(-L // S)
    P = n_pages + 3
    rng = np.random.default_rng(seed)
    bt = np.full((1, n_pages + 1), 0x7FFFFFFF, np.int32)
    bt[0, :n_pages] = rng.permutation(P)[:n_pages]
    cache = OracleCache("seq", kv, P, S, 1, D)
    W = n_pages + 1
    f1 = oracle_append(cache, bt, np.zeros(1, np.int32), np.array([L - T], np.int32),
                       K_bits[None, None, :L - T], V_bits[None, None, :L - T], W)
    f2 = oracle_append(cache, bt, np.array([L - T], np.int32), np.array([T], np.int32),
                       K_bits[None, None, L - T:], V_bits[None, None, L - T:], W)
    assert f1[0] == 0 and f2[0] == 0
    return cache, bt


@pytest.mark.parametrize("cfg,kw", [(1, {}), (3, dict(batch=2, lens=[20, 300])),
                                    (4, dict(batch=1))])
def test_m1_one_draft_is_decode(cfg, kw):
    if cfg == 4:
        kw = dict(lens=np.array([[33, 1, 512, 16, 17, 100, 5, 64]]))
    w = make_workload(cfg, **kw)
    cache, _ = oracle_fill(w)
    a = oracle_decode(cache, w.q, w.block_table, w.lens, w.sigma)
    b = oracle_decode_multi(cache, w.q[:, None], w.block_table, w.lens, w.sigma)
    assert np.array_equal(a, b[:, 0])


@pytest.mark.parametrize("T,L", [(2, 2), (4, 37), (8, 16), (8, 17), (5, 64)])
def test_m2_identical_keys_mean_over_visible_prefix(T, L):
    rng = np.random.default_rng(T * 100 + L)
    K = np.repeat(_bf16(rng.standard_normal((1, 64))), L, axis=0)
    V = _bf16(rng.standard_normal((L, 64)))
    cache, bt = _unit_cache(K, V, T)
    q = _bf16(rng.standard_normal((1, T, 1, 64)))
    out = oracle_decode_multi(cache, q, bt, np.array([L], np.int32), np.float32(0.125))
    Vf = bf16_to_f64(V)
    for t in range(T):
        n = L - T + t + 1
        assert np.max(np.abs(out[0, t, 0] - Vf[:n].mean(axis=0))) <= 1e-12, t


def test_m2_dominant_key_seen_only_from_its_position():
    """Key j is aligned with the query and large: drafts that see j return V[j]."""
    rng = np.random.default_rng(5)
    T, L, D = 6, 40, 64
    qv = np.zeros(D, np.float32); qv[3] = 1.0
    K = np.zeros((L, D), np.float32)
    j = L - T + 2                       # the third draft's own position
    K[j, 3] = 64.0                      # score 0.125 * 64 = 8 nats over every other key
    V = rng.standard_normal((L, D)).astype(np.float32)
    Kb, Vb = _bf16(K), _bf16(V)
    cache, bt = _unit_cache(Kb, Vb, T)
    q = np.repeat(_bf16(qv)[None, None, None], T, axis=1)
    out = oracle_decode_multi(cache, q, bt, np.array([L], np.int32), np.float32(0.125))
    Vf = bf16_to_f64(Vb)
    for t in range(T):
        n = L - T + t + 1
        if n > j:   # j visible: weight e^8 / (e^8 + n - 1) on V[j]
            wj = np.exp(8.0) / (np.exp(8.0) + n - 1)
            ref = wj * Vf[j] + (1 - wj) * (Vf[:n].sum(0) - Vf[j]) / (n - 1)
        else:       # all scores 0: plain mean
            ref = Vf[:n].mean(0)
        assert np.max(np.abs(out[0, t, 0] - ref)) <= 1e-12, t


def test_m3_causality_invariants():
    """Draft t ignores later drafts, and depends on its own token."""
    w = make_workload(2, batch=2, lens=[30, 129], q_len=5)
    cache, kv = oracle_fill(w)
    out = oracle_decode_multi(cache, w.q, w.block_table, w.lens, w.sigma)
    for b in range(w.B):
        L = int(w.lens[b])
        for t in range(w.q_len):
            # rewrite tokens L - T + t + 1 .. L - 1 (later drafts) with other values
            c2 = cache.copy()
            later = np.arange(L - w.q_len + t + 1, L)
            pages = w.block_table[b, later // w.S]
            c2.k[pages, :, later % w.S] ^= np.uint16(0x0040)
            c2.v[pages, :, later % w.S] ^= np.uint16(0x0040)
            o2 = oracle_decode_multi(c2, w.q, w.block_table, w.lens, w.sigma)
            assert np.array_equal(o2[b, t], out[b, t])
            if t + 1 < w.q_len:
                assert not np.array_equal(o2[b, t + 1], out[b, t + 1])
            # rewrite its own token: its output changes
            own = L - w.q_len + t
            c3 = cache.copy()
            c3.v[w.block_table[b, own // w.S], :, own % w.S] ^= np.uint16(0x0040)
            o3 = oracle_decode_multi(c3, w.q, w.block_table, w.lens, w.sigma)
            assert not np.array_equal(o3[b, t], out[b, t])
            assert np.array_equal(o3[b, :t], out[b, :t])


def _mp_attention(q, K, V, sigma):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(float(sigma)) * mpmath.fsum(mpmath.mpf(q[d]) * mpmath.mpf(K[t][d])
                                                for d in range(len(q))) for t in range(len(K))]
    m = max(s)
    e = [mpmath.exp(x - m) for x in s]
    den = mpmath.fsum(e)
    return [float(mpmath.fsum(e[t] * mpmath.mpf(V[t][d]) for t in range(len(K))) / den)
            for d in range(len(q))]


@pytest.mark.parametrize("S,L,T,D,Hq,Hkv", [(2, 9, 3, 4, 2, 1), (16, 20, 8, 8, 4, 2),
                                            (4, 8, 8, 4, 2, 2), (16, 33, 2, 8, 4, 1)])
def test_m4_brute_force_tiny(S, L, T, D, Hq, Hkv):
    rng = np.random.default_rng(S * 1000 + L * 10 + T)
    B = 2
    n_pages = -(-L // S)
    P = B * n_pages + 3
    perm = rng.permutation(P).astype(np.int32)
    W = n_pages + 1
    bt = np.full((B, W), 0x7FFFFFFF, np.int32)
    for b in range(B):
        bt[b, :n_pages] = perm[b * n_pages:(b + 1) * n_pages]
    K = _bf16(rng.standard_normal((B, Hkv, L, D)) * 2)
    V = _bf16(rng.standard_normal((B, Hkv, L, D)))
    q = _bf16(rng.standard_normal((B, T, Hq, D)))
    cache = OracleCache("seq", "bf16", P, S, Hkv, D)
    oracle_append(cache, bt, np.zeros(B, np.int32), np.full(B, L - T, np.int32),
                  K[:, :, :L - T], V[:, :, :L - T], W)
    oracle_append(cache, bt, np.full(B, L - T, np.int32), np.full(B, T, np.int32),
                  K[:, :, L - T:], V[:, :, L - T:], W)
    sigma = np.float32(1 / np.sqrt(D))
    out = oracle_decode_multi(cache, q, bt, np.full(B, L, np.int32), sigma)
    G = Hq // Hkv
    for b in range(B):
        for t in range(T):
            n = L - T + t + 1
            for hq in range(Hq):
                h = hq // G
                ref = _mp_attention(bf16_to_f64(q[b, t, hq]).tolist(),
                                    bf16_to_f64(K[b, h, :n]).tolist(),
                                    bf16_to_f64(V[b, h, :n]).tolist(), sigma)
                assert np.max(np.abs(out[b, t, hq] - np.array(ref))) <= 1e-13


@pytest.mark.parametrize("cfg,kw", [(2, dict(batch=2, lens=[8, 300])), (3, dict(batch=2, lens=[50, 77])),
                                    (4, dict(batch=1))])
def test_m5_torch_masked_attention(cfg, kw):
    """torch's scaled_dot_product_attention (CPU, fp64), bottom-right causal mask from torch.tril."""
    if cfg == 4:
        kw = dict(lens=np.array([[33, 8, 512, 16, 17, 100, 9, 64]]))
    T = 8 if cfg != 3 else 3
    w = make_workload(cfg, q_len=T, **kw)
    cache, kv = oracle_fill(w)
    out = oracle_decode_multi(cache, w.q, w.block_table, w.lens, w.sigma)
    for b in range(w.B):
        for h in range(w.Hkv):
            L = int(w.lens[b] if w.layout == "seq" else w.lens[b, h])
            if w.kv_dtype == "bf16":
                Kb, Vb = dense_tokens(kv[b], w.layout, h)
                K = torch.from_numpy(bf16_to_f64(Kb))
                V = torch.from_numpy(bf16_to_f64(Vb))
            else:   # FP8: the dequantised cache is the input; read it back through the table
                from oracle import gather_unit
                Kd, Vd = gather_unit(cache, w.block_table[b], h, L)
                K, V = torch.from_numpy(Kd), torch.from_numpy(Vd)
            qs = torch.from_numpy(bf16_to_f64(w.q[b, :, h * w.G:(h + 1) * w.G]))  # [T][G][D]
            mask = torch.ones(T, L, dtype=torch.bool).tril(diagonal=L - T)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qs.permute(1, 0, 2), K[None].expand(w.G, L, w.D), V[None].expand(w.G, L, w.D),
                attn_mask=mask, scale=float(w.sigma))          # [G][T][D]
            got = torch.from_numpy(out[b, :, h * w.G:(h + 1) * w.G]).permute(1, 0, 2)
            assert torch.max(torch.abs(got - ref)).item() <= 1e-12


def test_m6_degenerate_lengths_and_flags():
    """L < T: the first T - L drafts see nothing (zeros); flagged or empty units are zero."""
    rng = np.random.default_rng(8)
    T, D = 6, 64
    K = _bf16(rng.standard_normal((20, D)))
    V = _bf16(rng.standard_normal((20, D)))
    cache, bt = _unit_cache(K, V, 4)
    q = _bf16(rng.standard_normal((1, T, 1, D)))
    out = oracle_decode_multi(cache, q, bt, np.array([3], np.int32), np.float32(0.125))
    assert np.all(out[0, :3] == 0)              # drafts 0..2 would sit before position 0
    Vf = bf16_to_f64(V)
    assert np.max(np.abs(out[0, 3, 0] - Vf[0])) <= 1e-15   # one visible token: its value
    z = oracle_decode_multi(cache, q, bt, np.array([0], np.int32), np.float32(0.125))
    assert np.all(z == 0)
    f = oracle_decode_multi(cache, q, bt, np.array([20], np.int32), np.float32(0.125),
                            flags=np.array([1], np.uint32))
    assert np.all(f == 0)
