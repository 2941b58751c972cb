"""Test helper: build the oracle's cache for a workload by replaying its appends.

A workload's cache is produced the way a decode loop would produce it: one bulk
append of the first L-1 tokens of each sequence into empty pages, then one
append of the step's new token.  Only oracle code and the shared input
generator are used here.
"""
import numpy as np

from oracle import OracleCache, oracle_append


def seq_rows(w, b):
    """Sub-batch views (batch of one) of sequence b's table and lengths."""
    bt = w.block_table[b:b + 1]
    if w.layout == "seq":
        return bt, np.array([w.lens[b]], np.int32)
    return bt, w.lens[b:b + 1]


def oracle_fill(w, seqs=None, cache=None):
    """Replay the appends of sequences `seqs` (default: all) into an oracle cache.

    Returns (cache, kv) where kv[b] = the generator's draws for sequence b.
    """
    if cache is None:
        cache = OracleCache(w.layout, w.kv_dtype, w.P, w.S, w.Hkv, w.D)
    seqs = range(w.B) if seqs is None else seqs
    kv = {}
    for b in seqs:
        k_hist, v_hist, k_new, v_new, n_hist = w.seq_kv(b)
        kv[b] = (k_hist, v_hist, k_new, v_new, n_hist)
        bt, _ = seq_rows(w, b)
        if w.layout == "seq":
            zero = np.zeros(1, np.int32)
            n1 = np.array([n_hist[0]], np.int32)
            one = np.ones(1, np.int32)
        else:
            zero = np.zeros((1, w.Hkv), np.int32)
            n1 = n_hist[None, :].astype(np.int32)
            one = np.ones((1, w.Hkv), np.int32)
        f1 = oracle_append(cache, bt, zero, n1, k_hist[None], v_hist[None], w.W)
        f2 = oracle_append(cache, bt, n1, one, k_new[None], v_new[None], w.W)
        assert f1[0] == 0 and f2[0] == 0
    return cache, kv


def dense_tokens(kv_b, layout, h):
    """The L tokens of (sequence, KV head h) in order, as bf16 bits [L][D] (K, V)."""
    k_hist, v_hist, k_new, v_new, n_hist = kv_b
    n = int(n_hist[h])
    K = np.concatenate([k_hist[h, :n], k_new[h]], axis=0)
    V = np.concatenate([v_hist[h, :n], v_new[h]], axis=0)
    return K, V
