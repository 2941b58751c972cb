"""Seeded synthetic inputs for paged decode attention.

This module only draws inputs: lengths, page assignment, tags, queries and
the K/V tokens of each sequence.  It holds none of the method's arithmetic and
is shared by the tests, the bench and the smoke check (both the HIP path and
the oracle read the same draws).

Shapes follow the five workloads of this library:

  1  tiny:        B 4,  8/2 heads, D 64,  S 16, L in {37, 100, 256, 511},
                  BF16, SEQ, pool of 128 pages, W 32
  2  llama8b:     B 32, 32/8 heads, D 128, L ~ U{1024..8192}, BF16, SEQ, W 512
  3  llama8b-fp8: B 64, 32/8 heads, D 128, L ~ U{4096..16384}, FP8, SEQ, W 1024,
                  1% of the used table entries carry a stale expected tag
  4  headwise:    B 16, 32/8 heads, D 128, L(b,h) = 32768 / f, f ~ U{1, 8, 64}
                  per (sequence, KV head), BF16, HEAD layout, W 2048
  5  70b-fp8:     B 64, 64/8 heads, D 128, L = 32768, FP8, SEQ, W 2048

Recipe (one numpy PCG64 stream per workload, seed = workload number unless
given):
  1. lengths (and the per-head factor f for workload 4);
  2. a random permutation of the P physical pages, P = used pages + 64 spare
     (128 for workload 1), dealt to the table entries in unit order;
     unused entries hold 0x7FFFFFFF;
  3. uint32 page tags, uniform;
  4. Q ~ N(0, 1) fp32, rounded to BF16 (round to nearest even);
  5. the stale-entry choice: round(frac * used entries) entries, uniform
     without replacement, whose expected tag is the page tag minus 1.
K and V of sequence b come from the child stream SeedSequence(seed).spawn(B)[b]
so that any one sequence can be regenerated on its own: per KV head h, K
history [L-1][D], V history, then the new token's K and V (SEQ layout draws
all heads at once in that order).  All values are N(0, 1) fp32 rounded to BF16.
A decode step appends the new token, then attends all L tokens.

Multi-query workloads (q_len T > 1, speculative verification) draw the same
way with T in place of the single new token: per KV head a history of L - T
tokens, then the T draft tokens; queries are [B][T][Hq][D], drawn in step 4
instead of the [B][Hq][D] ones.  With T = 1 every draw is the one above.

Magnitudes (kv_mag, for range tests of the FP8 cache): K and V may be
multiplied, before the BF16 rounding, by a constant, by a factor drawn per
logical page of each unit (10^U(lo, hi), "pages"), or by a factor that grows
along the unit (10^(lo + (hi - lo) * page / pages), "ramp").  The factors come
after all other draws of the sequence's stream, so the N(0, 1) draws are the
same with or without them.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

UNUSED_ENTRY = 0x7FFFFFFF


@dataclass
class Workload:
    cfg_id: int
    name: str
    layout: str                 # "seq" | "head"
    kv_dtype: str               # "bf16" | "fp8"
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    W: int
    P: int
    sigma: np.float32
    lens: np.ndarray            # int32 [B] or [B][Hkv]: tokens attended
    block_table: np.ndarray     # int32 [B][W] or [B][Hkv][W]
    page_tags: np.ndarray       # uint32 [P]
    expected_tags: np.ndarray   # uint32, shape of block_table
    stale: np.ndarray           # bool, shape of block_table
    q: np.ndarray               # uint16 bf16 bits [B][Hq][D], or [B][T][Hq][D] when q_len > 1
    seed: int = 0
    q_len: int = 1              # T: query (draft) tokens per sequence, the last T of each unit
    extra: dict = field(default_factory=dict)
    kv_mag: dict = None         # {"k"|"v": float | ("pages"|"ramp", lo, hi)} magnitudes

    @property
    def G(self):
        return self.Hq // self.Hkv

    def n_pages_used(self):
        return int(np.sum(-(-self.lens.astype(np.int64) // self.S)))

    def seq_kv(self, b):
        """K/V draws of sequence b (bf16 bits).

        Returns (k_hist, v_hist, k_new, v_new, n_hist) with k_hist/v_hist
        [Hkv][max_h(L-T)][D] (rows past a head's own L-T are zero padding),
        k_new/v_new [Hkv][T][D] and n_hist int32 [Hkv] = L(b, h) - T.
        """
        rng = np.random.default_rng(np.random.SeedSequence(self.seed).spawn(self.B)[b])
        T = self.q_len
        if self.layout == "seq":
            L = int(self.lens[b])
            n_hist = np.full(self.Hkv, max(L - T, 0), np.int32)
            kh = rng.standard_normal((self.Hkv, max(L - T, 0), self.D), dtype=np.float32)
            vh = rng.standard_normal((self.Hkv, max(L - T, 0), self.D), dtype=np.float32)
            kn = rng.standard_normal((self.Hkv, T, self.D), dtype=np.float32)
            vn = rng.standard_normal((self.Hkv, T, self.D), dtype=np.float32)
        else:
            n_hist = np.maximum(self.lens[b].astype(np.int32) - T, 0)
            nmax = int(n_hist.max()) if n_hist.size else 0
            kh = np.zeros((self.Hkv, nmax, self.D), np.float32)
            vh = np.zeros_like(kh)
            kn = np.zeros((self.Hkv, T, self.D), np.float32)
            vn = np.zeros_like(kn)
            for h in range(self.Hkv):
                n = int(n_hist[h])
                kh[h, :n] = rng.standard_normal((n, self.D), dtype=np.float32)
                vh[h, :n] = rng.standard_normal((n, self.D), dtype=np.float32)
                kn[h] = rng.standard_normal((T, self.D), dtype=np.float32)
                vn[h] = rng.standard_normal((T, self.D), dtype=np.float32)
        if self.kv_mag:
            for which, (hist, new) in (("k", (kh, kn)), ("v", (vh, vn))):
                spec = self.kv_mag.get(which)
                if spec is None:
                    continue
                for h in range(self.Hkv):
                    n = int(n_hist[h])
                    f = _magnitudes(spec, n + T, self.S, rng)
                    hist[h, :n] *= f[:n, None]
                    new[h] *= f[n:, None]
        return (to_bf16_bits(kh), to_bf16_bits(vh), to_bf16_bits(kn), to_bf16_bits(vn), n_hist)


def _magnitudes(spec, L, S, rng):
    """Per-token fp32 factors of one unit of L tokens (see kv_mag)."""
    if not isinstance(spec, tuple):
        return np.full(L, spec, np.float32)
    kind, lo, hi = spec
    pages = max(-(-L // S), 1)
    if kind == "pages":
        e = rng.uniform(lo, hi, size=pages)
    elif kind == "ramp":
        e = lo + (hi - lo) * np.arange(pages) / max(pages - 1, 1)
    else:
        raise ValueError(kind)
    return np.repeat((10.0 ** e).astype(np.float32), S)[:L]


def to_bf16_bits(x):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


CONFIG_NAMES = {1: "tiny", 2: "llama8b-bf16", 3: "llama8b-fp8-tags", 4: "headwise-bf16",
                5: "70b-fp8-32k"}


def make_workload(cfg_id, *, batch=None, lens=None, seed=None, stale_frac=None,
                  spare_pages=64, table_width=None, q_len=1, heads=None, kv=None, layout=None,
                  head_dim=None, kv_mag=None, sigma=None):
    """Draw workload `cfg_id` (1..5).

    batch / lens / table_width override the workload's own sizes for reduced
    parity cases; stale_frac overrides the fraction of stale expected tags
    (workload 3 defaults to 0.01, the others to 0); q_len > 1 makes the step
    a multi-query step of q_len query tokens (speculative verification: up to
    8 drafts; chunked prefill: a chunk of q_len prompt tokens);
    heads = (Hq, Hkv) overrides the head counts (edge cases of the grouping);
    kv ("bf16" | "fp8"), layout ("seq" | "head") and head_dim (64 | 128)
    override the cache format, for the combinations no named workload uses;
    kv_mag scales K and V (see the module notes) and sigma overrides the
    softmax scale 1/sqrt(D).
    The draws keep their order; their sizes follow the overridden shapes.
    """
    if int(q_len) < 1:
        raise ValueError("q_len must be at least 1")
    seed = cfg_id if seed is None else seed
    rng = np.random.default_rng(seed)
    spec = {
        1: dict(layout="seq", kv="bf16", B=4, Hq=8, Hkv=2, D=64, W=32),
        2: dict(layout="seq", kv="bf16", B=32, Hq=32, Hkv=8, D=128, W=512),
        3: dict(layout="seq", kv="fp8", B=64, Hq=32, Hkv=8, D=128, W=1024),
        4: dict(layout="head", kv="bf16", B=16, Hq=32, Hkv=8, D=128, W=2048),
        5: dict(layout="seq", kv="fp8", B=64, Hq=64, Hkv=8, D=128, W=2048),
    }[cfg_id]
    S = 16
    B = spec["B"] if batch is None else int(batch)
    W = spec["W"] if table_width is None else int(table_width)
    Hkv, Hq, D = spec["Hkv"], spec["Hq"], spec["D"]
    if heads is not None:
        Hq, Hkv = int(heads[0]), int(heads[1])
    spec = dict(spec, kv=kv or spec["kv"], layout=layout or spec["layout"])
    if head_dim is not None:
        D = int(head_dim)

    # 1. lengths
    if lens is not None:
        L = np.asarray(lens, dtype=np.int32)
    elif cfg_id == 1:
        L = np.array([37, 100, 256, 511], np.int32)[:B]
    elif cfg_id == 2:
        L = rng.integers(1024, 8192, size=B, endpoint=True).astype(np.int32)
    elif cfg_id == 3:
        L = rng.integers(4096, 16384, size=B, endpoint=True).astype(np.int32)
    elif cfg_id == 4:
        f = rng.choice(np.array([1, 8, 64]), size=(B, Hkv))
        L = (32768 // f).astype(np.int32)
    else:
        L = np.full(B, 32768, np.int32)
    if spec["layout"] == "head" and L.ndim == 1:
        L = np.repeat(L[:, None], Hkv, axis=1)
    B = L.shape[0]
    if q_len > 1 and np.any(L < q_len):
        raise ValueError("every unit of a multi-query step holds its q_len draft tokens")

    # 2. pages
    n_rows = L.reshape(-1)
    need = -(-n_rows.astype(np.int64) // S)
    used = int(need.sum())
    P = 128 if (cfg_id == 1 and lens is None and batch is None) else used + spare_pages
    P = max(P, used)
    perm = rng.permutation(P).astype(np.int32)
    bt_rows = np.full((n_rows.size, W), UNUSED_ENTRY, np.int32)
    k = 0
    for r, n in enumerate(need):
        n = int(min(n, W))
        bt_rows[r, :n] = perm[k:k + n]
        k += int(need[r])
    block_table = bt_rows.reshape(L.shape + (W,))

    # 3. tags
    page_tags = rng.integers(0, 2 ** 32, size=P, dtype=np.uint64).astype(np.uint32)

    # 4. queries
    qshape = (B, Hq, D) if q_len == 1 else (B, int(q_len), Hq, D)
    q = to_bf16_bits(rng.standard_normal(qshape, dtype=np.float32))

    # 5. expected tags, some stale
    frac = (0.01 if cfg_id == 3 else 0.0) if stale_frac is None else stale_frac
    exp_rows = np.zeros_like(bt_rows, dtype=np.uint32)
    used_idx = []
    for r, n in enumerate(need):
        n = int(min(n, W))
        exp_rows[r, :n] = page_tags[bt_rows[r, :n]]
        used_idx.extend((r, i) for i in range(n))
    stale_rows = np.zeros(bt_rows.shape, bool)
    n_stale = int(round(frac * len(used_idx)))
    if n_stale:
        pick = rng.choice(len(used_idx), size=n_stale, replace=False)
        for j in pick:
            r, i = used_idx[j]
            stale_rows[r, i] = True
            exp_rows[r, i] = np.uint32((int(exp_rows[r, i]) - 1) % 2 ** 32)

    return Workload(
        cfg_id=cfg_id, name=CONFIG_NAMES[cfg_id], layout=spec["layout"], kv_dtype=spec["kv"],
        B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, W=W, P=P,
        sigma=np.float32(1.0 / np.sqrt(D)) if sigma is None else np.float32(sigma),
        lens=L, block_table=block_table, page_tags=page_tags,
        expected_tags=exp_rows.reshape(block_table.shape),
        stale=stale_rows.reshape(block_table.shape), q=q, seed=seed, q_len=int(q_len),
        kv_mag=kv_mag)
