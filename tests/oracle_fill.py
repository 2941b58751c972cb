"""Test helper: build the oracle's cache for a workload by replaying its appends.

A workload's cache is produced the way a decode loop would produce it: one bulk
append of the first L-T tokens of each sequence into empty pages, then one
append of the step's T new tokens (T = 1, or the draft tokens of a multi-query
step).  Only oracle code and the shared input
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


def oracle_fill(w, seqs=None, cache=None, step_tags=True):
    """Replay the appends of sequences `seqs` (default: all) into an oracle cache.

    The bulk fill writes the history into fresh pages; the step's append goes
    through the expected tags (with step_tags), as the GPU step does: a page
    whose entry is stale is left alone.
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
        # the step appends q_len tokens to every unit that is not empty (an
        # empty unit has neither history nor step tokens)
        if w.layout == "seq":
            zero = np.zeros(1, np.int32)
            n1 = np.array([n_hist[0]], np.int32)
            one = np.full(1, w.q_len if int(w.lens[b]) > 0 else 0, np.int32)
        else:
            zero = np.zeros((1, w.Hkv), np.int32)
            n1 = n_hist[None, :].astype(np.int32)
            one = np.where(w.lens[b:b + 1] > 0, w.q_len, 0).astype(np.int32)
        f1 = oracle_append(cache, bt, zero, n1, k_hist[None], v_hist[None], w.W)
        tags = dict(expected_tags=w.expected_tags[b:b + 1], page_tags=w.page_tags) \
            if step_tags else {}
        f2 = oracle_append(cache, bt, n1, one, k_new[None], v_new[None], w.W, **tags)
        assert f1[0] == 0 and (f2[0] & ~np.uint32(1)) == 0
    return cache, kv


def dense_tokens(kv_b, layout, h):
    """The L tokens of (sequence, KV head h) in order, as bf16 bits [L][D] (K, V)."""
    k_hist, v_hist, k_new, v_new, n_hist = kv_b
    n = int(n_hist[h])
    K = np.concatenate([k_hist[h, :n], k_new[h]], axis=0)
    V = np.concatenate([v_hist[h, :n], v_new[h]], axis=0)
    return K, V


def oracle_sequence(w, b, with_mass=False, with_pools=True):
    """Oracle result of sequence b alone, on a compact local pool.

    The sequence's pages are renumbered 0..n-1 (the result does not depend on
    physical page ids: page-permutation invariance is pinned separately).
    Returns dict(pages=global page ids [n], k, v = local logical pools [n][H][S][D],
    k_scale, v_scale = [n][H] or None, out = fp64 [Hq][D], or [T][Hq][D] for a
    multi-query workload (unflagged result)); with_mass adds mass = {h: the
    step's attention mass per token [L]} (decode workloads); without
    with_pools the pools and scales are left out (None).
    """
    from oracle import oracle_attention_mass, oracle_decode, oracle_decode_multi

    rows = w.block_table[b:b + 1]
    lens = w.lens[b:b + 1]
    need = -(-lens.astype(np.int64) // w.S)
    flat_rows = rows.reshape(-1, w.W)
    flat_need = need.reshape(-1)
    pages = np.concatenate([flat_rows[r, :min(int(n), w.W)] for r, n in enumerate(flat_need)])
    local = np.full(flat_rows.shape, 0x7FFFFFFF, np.int32)
    k = 0
    for r, n in enumerate(flat_need):
        n = int(min(n, w.W))
        local[r, :n] = np.arange(k, k + n, dtype=np.int32)
        k += n
    local = local.reshape(rows.shape)
    n_pages = max(len(pages), 1)
    sub = _SubWorkload(w, b, local, n_pages)
    cache, _ = oracle_fill(sub, seqs=[0])
    if w.q_len == 1:
        out = oracle_decode(cache, w.q[b:b + 1], local, lens, w.sigma)[0]
    else:
        out = oracle_decode_multi(cache, w.q[b:b + 1], local, lens, w.sigma)[0]
    r = dict(pages=pages, k=None, v=None, k_scale=None, v_scale=None, out=out)
    if with_pools:
        r.update(k=cache.k[:len(pages)], v=cache.v[:len(pages)],
                 k_scale=None if cache.k_scale is None else cache.k_scale[:len(pages)],
                 v_scale=None if cache.v_scale is None else cache.v_scale[:len(pages)])
    if with_mass:
        m = oracle_attention_mass(cache, w.q[b:b + 1], local, lens, w.sigma)
        r["mass"] = {h: m[(0, h)] for (_, h) in m}
    return r


class _SubWorkload:
    """Sequence b of a workload seen as a batch of one with a local page table."""

    def __init__(self, w, b, local_table, n_pages):
        self._w, self._b = w, b
        self.layout, self.kv_dtype, self.S, self.W = w.layout, w.kv_dtype, w.S, w.W
        self.Hkv, self.D, self.P, self.B = w.Hkv, w.D, n_pages, 1
        self.block_table = local_table
        self.lens = w.lens[b:b + 1]
        self.q_len = w.q_len
        # the local pages carry their global pages' tags; entries keep theirs
        self.expected_tags = np.zeros(local_table.shape, np.uint32)
        self.page_tags = np.zeros(n_pages, np.uint32)
        if w.page_tags is not None:
            rows = w.block_table[b:b + 1].reshape(-1, w.W)
            loc = local_table.reshape(-1, w.W)
            exp = w.expected_tags[b:b + 1].reshape(-1, w.W)
            for r in range(rows.shape[0]):
                used = loc[r] != 0x7FFFFFFF
                self.expected_tags.reshape(-1, w.W)[r, used] = exp[r, used]
                self.page_tags[loc[r, used]] = w.page_tags[rows[r, used]]

    def seq_kv(self, _):
        return self._w.seq_kv(self._b)


def _workers(n):
    import os

    return max(1, min(16, len(os.sched_getaffinity(0)), n))


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _pool(workers):
    """A spawn pool whose workers run one BLAS/OpenMP thread each (one worker per
    core; threaded BLAS in every worker would oversubscribe the cores).  The
    workers start with the pool, under the environment set here."""
    import multiprocessing
    import os
    from concurrent.futures import ProcessPoolExecutor

    saved = {k: os.environ.get(k) for k in _THREAD_VARS}
    for k in _THREAD_VARS:
        os.environ[k] = "1"
    try:
        # spawn: a forked child of a process with live OpenMP/torch thread pools can deadlock
        ex = ProcessPoolExecutor(workers, mp_context=multiprocessing.get_context("spawn"))
        list(ex.map(_ready, range(workers)))   # start every worker now, under this environment
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return ex


def _ready(_):
    return True


def _run(ex, w, seqs, with_mass, with_pools):
    n = len(seqs)
    if ex is None:
        return {b: oracle_sequence(w, b, with_mass, with_pools) for b in seqs}
    return dict(zip(seqs, ex.map(oracle_sequence, [w] * n, seqs, [with_mass] * n,
                                 [with_pools] * n)))


def oracle_sequences_parallel(w, seqs, workers=None, with_mass=False, with_pools=True):
    """oracle_sequence for several sequences in a process pool."""
    seqs = list(seqs)
    workers = workers or _workers(len(seqs))
    if workers == 1:
        return _run(None, w, seqs, with_mass, with_pools)
    with _pool(workers) as ex:
        return _run(ex, w, seqs, with_mass, with_pools)


def oracle_chunks(w, seqs, size=16, with_mass=False, with_pools=True):
    """oracle_sequence over consecutive chunks of `size` sequences, on one process
    pool (a generator: each chunk's pools are dropped once the caller moves on)."""
    seqs = list(seqs)
    workers = _workers(size)
    ex = _pool(workers) if workers > 1 else None
    try:
        for i in range(0, len(seqs), size):
            yield _run(ex, w, seqs[i:i + size], with_mass, with_pools)
    finally:
        if ex is not None:
            ex.shutdown()
