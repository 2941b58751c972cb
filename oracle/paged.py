"""Plain, slow, fp64 reference for paged decode attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg; never by the product path.  It shares no code with
the HIP library and reads the cache through its own logical layout.

What it computes, and where the pages say so:
  * Paged KV cache: the cache is split into fixed-size pages that are assigned
    on demand; a decode step revisits every cached K/V of its sequence
    ("How we built the most efficient inference engine for Cloudflare's
    network", section "Batching to feed the Tensor Cores", KV-cache paragraph).
  * Block table of integer page indices; one table per (sequence, head) lets
    heads keep different numbers of tokens ("Making Workers AI faster and more
    efficient" -- KV cache compression page, section "KV cache compression goes
    open source", the block-table paragraph).
  * FP8 e4m3 KV cache instead of BF16 ("Cloudflare quantizes Kimi and GLM
    caches for 41% faster inference", KV cache quantization paragraph).
  * Page-tag integrity check: each physical page carries a tag that changes on
    reallocation; the server records the (page, tag) pairs a request expects;
    the pairs are checked in a separate batch validation before decode reads
    the cache, and a mismatch aborts the request (same page, integrity-check
    paragraph).

Readings taken where the pages are silent (each is also in the design notes):
  R1 Logical layout: SEQ pools are [P][Hkv][S][D] with a [B][W] table and [B]
     lengths; HEAD pools are [P][S][D] with a [B][Hkv][W] table and [B][Hkv]
     lengths.  Token t of a unit lives at page table[t // S], slot t % S.
  R2 FP8 scales: one fp32 scale per (physical page, KV head), separate for K
     and V, kept equal to fl32(amax / 448) over every value written to that
     page-head since the page was last started fresh.
  R3 Quantisation: code = e4m3_rne_sat(fl32(x / s)); fl32 is IEEE binary32
     division (numpy float32), then an exact round-to-nearest-even.
  R4 Appending into a partly filled page: when the new values raise the scale
     from s_old to s_new, the codes already in the page are re-quantised as
     e4m3_rne_sat(fl32(fl32(dec(c) * s_old) / s_new)).  A page whose first
     written slot in a call is slot 0 is fresh: its old scale is ignored.
  R5 Append refuses out-of-range page ids (flag bit 1) and writes past
     table_width * S (flag bit 2).  Given the tags a request expects, it
     writes a page only through an entry whose expected tag is the page's
     current tag, and otherwise leaves the page alone and sets flag bit 0:
     the check exists to protect requests that share GPU memory, and a
     stale entry names a page that may now hold another request's tokens
     (integrity-check paragraph).  Without expected tags it checks none.
  R6 Validation flags, per sequence b, OR-ed over its units: bit 0 a tag
     mismatch, bit 1 a page id outside [0, P) (its tag is then not compared),
     bit 2 a length above table_width * S (entries checked up to the width).
     Only the ceil(L / S) entries a decode would read are checked.
  R7 Decode: query head hq uses KV head hq // (Hq / Hkv); scores are
     sigma * q . k over all L tokens; softmax with the max subtracted; a
     flagged sequence, or a unit with L = 0, yields exact zeros.
  R8 Multi-query decode (speculative verification: the target model checks
     all draft tokens of a sequence in one forward pass -- "Making Workers AI
     faster and more efficient", section "Speculative decoding: predicting
     more than one token"; the extra-large-models write-up, part 4 on
     speculative decoding).  The T drafts are the last T tokens of each unit,
     appended before the call; draft t (0-based) sits at position L - T + t
     and attends tokens 0 .. L - T + t: the whole earlier cache, itself, and
     the drafts before it.  A draft with no such token (L - T + t < 0) yields
     zeros, as a flagged sequence does.
  R9 Eviction score (KV-compression page, section "KV cache compression goes
     open source": evict the KV entries with the lowest accumulated past
     attention, like a least-frequently-used policy; the per-head block table
     lets heads be compressed at different rates).  The score of a cached
     token of a (sequence, KV head) grows at each decode step by the softmax
     weight the step puts on it, summed over the G query heads of the group.
     Scores are fp32, one per physical (page, head, slot), so they travel with
     the page.  Flagged sequences and slots past L are not updated.
  R10 Compaction after eviction: the tokens a unit keeps (strictly increasing
     positions) are written, in order, from position 0 into the pages of a new
     table.  BF16 values are copied.  FP8 values are first decoded under their
     old page scale, x = fl32(dec(c) * s_old), then quantised into the new
     page as an append of fresh pages does (R2, R3): s = fl32(amax / 448) over
     the page's x, codes RNE(sat(fl32(x / s))).  Scores are copied with their
     tokens.
"""
import numpy as np

from .codecs import (
    bf16_to_f64,
    e4m3_from_f32_rne_sat,
    e4m3_to_f64,
)

FLAG_TAG_MISMATCH = 1
FLAG_PAGE_OOB = 2
FLAG_LEN_OVERFLOW = 4
E4M3_MAX_F32 = np.float32(448.0)


class OracleCache:
    """Logical cache state: pools indexed [page][head][slot][dim].

    HEAD layout pools carry a head axis of length 1 so that both layouts share
    one indexing rule inside the oracle.
    """

    def __init__(self, layout, kv_dtype, num_pages, page_size, num_kv_heads, head_dim):
        assert layout in ("seq", "head") and kv_dtype in ("bf16", "fp8")
        self.layout, self.kv_dtype = layout, kv_dtype
        self.P, self.S, self.Hkv, self.D = num_pages, page_size, num_kv_heads, head_dim
        ph = num_kv_heads if layout == "seq" else 1
        if kv_dtype == "bf16":
            self.k = np.full((num_pages, ph, page_size, head_dim), 0x7FC0, np.uint16)
            self.v = np.full_like(self.k, 0x7FC0)
            self.k_scale = self.v_scale = None
        else:
            self.k = np.full((num_pages, ph, page_size, head_dim), 0x7F, np.uint8)
            self.v = np.full_like(self.k, 0x7F)
            self.k_scale = np.full((num_pages, ph), np.nan, np.float32)
            self.v_scale = np.full((num_pages, ph), np.nan, np.float32)

    def copy(self):
        c = OracleCache.__new__(OracleCache)
        c.__dict__.update(self.__dict__)
        c.k, c.v = self.k.copy(), self.v.copy()
        if self.k_scale is not None:
            c.k_scale, c.v_scale = self.k_scale.copy(), self.v_scale.copy()
        return c


def units(layout, batch, num_kv_heads):
    """(b, kv head, table-row index, pool head index) for every attention unit.

    SEQ: one table row per sequence, shared by all KV heads.
    HEAD: one table row per (sequence, KV head); the pool has no head axis.
    """
    out = []
    for b in range(batch):
        for h in range(num_kv_heads):
            if layout == "seq":
                out.append((b, h, (b,), h))
            else:
                out.append((b, h, (b, h), 0))
    return out


# --------------------------------------------------------------- append
def _quantise(values_f32, scale):
    """R3: codes of fp32 values under one fp32 scale (scale 0 -> all +0)."""
    if scale == 0:
        return np.zeros(values_f32.shape, np.uint8)
    q = (values_f32.astype(np.float32) / np.float32(scale)).astype(np.float32)
    return e4m3_from_f32_rne_sat(q)


def _append_fp8_page(pool, scales, pid, ph, first_slot, slots, new_bits):
    """R2/R4 for one (page, head) and one of K or V.

    new_bits: bf16 bit patterns [len(slots)][D] written at `slots`, which are
    consecutive and start at first_slot.
    """
    x = bf16_to_f64(new_bits).astype(np.float32)        # exact: bf16 is a subset of fp32
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s_cand = np.float32(amax / E4M3_MAX_F32)            # fl32(amax / 448)
    s_old = np.float32(0) if first_slot == 0 else scales[pid, ph]
    s_new = max(s_old, s_cand)
    if s_new > s_old and first_slot > 0:
        old = e4m3_to_f64(pool[pid, ph, :first_slot]).astype(np.float32)   # exact
        back = (old * s_old).astype(np.float32)          # fl32(dec(c) * s_old)
        pool[pid, ph, :first_slot] = _quantise(back, s_new)
    pool[pid, ph, slots] = _quantise(x, s_new)
    scales[pid, ph] = s_new


def _append_whole_pages(c, table, i, whole, row, b, h, ph, t, k_new, v_new, flags,
                        expected_tags, page_tags):
    """R2-R5 for `whole` whole pages (table entries i ...), each started afresh
    at slot 0 by this call: per page, s = fl32(amax / 448) and codes
    e4m3_rne_sat(fl32(x / s)) (no earlier codes to re-quantise), the same
    arithmetic as _append_fp8_page, done for all the pages at once.  Returns
    the tokens handled, or 0 (the caller then goes page by page) when two
    entries of the run name the same page."""
    S, P = c.S, c.P
    pids = np.asarray(table[i:i + whole], dtype=np.int64)
    ok = (pids >= 0) & (pids < P)
    if not ok.all():
        flags[b] |= FLAG_PAGE_OOB
    if expected_tags is not None:
        exp = np.asarray(expected_tags[row][i:i + whole])
        tag_ok = ok.copy()
        tag_ok[ok] = exp[ok] == page_tags[pids[ok]]
        if (ok & ~tag_ok).any():
            flags[b] |= FLAG_TAG_MISMATCH
        ok = tag_ok
    sel = pids[ok]
    if len(np.unique(sel)) != len(sel):
        return 0
    for pool, scales, src in ((c.k, c.k_scale, k_new), (c.v, c.v_scale, v_new)):
        bits = src[b, h, t:t + whole * S].reshape(whole, S, -1)[ok]
        if c.kv_dtype == "bf16":
            pool[sel, ph] = bits
            continue
        x = bf16_to_f64(bits).astype(np.float32)                       # exact
        amax = np.max(np.abs(x), axis=(1, 2)).astype(np.float32)
        scale = (amax / E4M3_MAX_F32).astype(np.float32)              # fl32(amax / 448)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (x / scale[:, None, None]).astype(np.float32)           # fl32(x / s)
        codes = e4m3_from_f32_rne_sat(q)
        pool[sel, ph] = np.where(scale[:, None, None] == 0, np.uint8(0), codes)
        scales[sel, ph] = scale
    return whole * S


def oracle_append(cache, block_table, lens_old, n_new, k_new, v_new, table_width,
                  expected_tags=None, page_tags=None):
    """Write n_new[u] tokens per unit at positions lens_old[u] ... .

    block_table: int32 [B][W] (SEQ) or [B][Hkv][W] (HEAD)
    lens_old, n_new: int32 [B] (SEQ) or [B][Hkv] (HEAD)
    k_new, v_new: bf16 bits uint16 [B][Hkv][n_max][D]
    expected_tags (the table's shape) with page_tags (uint32 [P]): R5's gate.
    Updates `cache` in place and returns the per-sequence flags (uint32 [B]).
    """
    c = cache
    B, Hkv = k_new.shape[0], k_new.shape[1]
    S, W, P = c.S, table_width, c.P
    flags = np.zeros(B, np.uint32)
    for (b, h, row, ph) in units(c.layout, B, Hkv):
        table = block_table[row]
        pos0, n = int(lens_old[row]), int(n_new[row])
        if pos0 + n > W * S:
            flags[b] |= FLAG_LEN_OVERFLOW
        n_ok = max(0, min(pos0 + n, W * S) - pos0)
        t = 0
        while t < n_ok:                       # one page at a time
            pos = pos0 + t
            i, slot0 = pos // S, pos % S
            whole = (n_ok - t) // S if slot0 == 0 else 0
            if whole >= 2:                    # a run of whole fresh pages, all at once
                done = _append_whole_pages(c, table, i, whole, row, b, h, ph, t, k_new, v_new,
                                           flags, expected_tags, page_tags)
                if done:
                    t += done
                    continue
            cnt = min(S - slot0, n_ok - t)
            pid = int(table[i])
            if not (0 <= pid < P):
                flags[b] |= FLAG_PAGE_OOB
                t += cnt
                continue
            if expected_tags is not None and expected_tags[row][i] != page_tags[pid]:
                flags[b] |= FLAG_TAG_MISMATCH        # the page is someone else's now
                t += cnt
                continue
            slots = np.arange(slot0, slot0 + cnt)
            for pool, scales, src in ((c.k, c.k_scale, k_new), (c.v, c.v_scale, v_new)):
                bits = src[b, h, t:t + cnt]
                if c.kv_dtype == "bf16":
                    pool[pid, ph, slots] = bits
                else:
                    _append_fp8_page(pool, scales, pid, ph, slot0, slots, bits)
            t += cnt
    return flags


# ------------------------------------------------------------- validate
def oracle_validate(layout, num_pages, page_size, block_table, lens, page_tags,
                    expected_tags, table_width):
    """R6.  expected_tags None is the no-op tracker: only bits 1 and 2."""
    B = block_table.shape[0]
    Hkv = 1 if layout == "seq" else block_table.shape[1]
    flags = np.zeros(B, np.uint32)
    for (b, h, row, _) in units(layout, B, Hkv):
        L = int(lens[row])
        if L > table_width * page_size:
            flags[b] |= FLAG_LEN_OVERFLOW
        n_pages = -(-min(L, table_width * page_size) // page_size)
        for i in range(n_pages):
            pid = int(block_table[row][i])
            if not (0 <= pid < num_pages):
                flags[b] |= FLAG_PAGE_OOB
            elif expected_tags is not None and expected_tags[row][i] != page_tags[pid]:
                flags[b] |= FLAG_TAG_MISMATCH
    return flags


# --------------------------------------------------------------- decode
def gather_unit(cache, table_row, ph, L):
    """K-hat, V-hat of one unit as dense fp64 [L][D] (the M x N view of one head)."""
    S = cache.S
    n_pages = -(-L // S)
    pages = np.asarray(table_row[:n_pages], dtype=np.int64)
    kb = cache.k[pages, ph].reshape(n_pages * S, cache.D)[:L]
    vb = cache.v[pages, ph].reshape(n_pages * S, cache.D)[:L]
    if cache.kv_dtype == "bf16":
        return bf16_to_f64(kb), bf16_to_f64(vb)
    ks = np.repeat(cache.k_scale[pages, ph].astype(np.float64), S)[:L]
    vs = np.repeat(cache.v_scale[pages, ph].astype(np.float64), S)[:L]
    return e4m3_to_f64(kb) * ks[:, None], e4m3_to_f64(vb) * vs[:, None]


def attention_f64(q, K, V, sigma):
    """Textbook single-query softmax attention in fp64: returns (o, weights)."""
    z = float(sigma) * (K @ q)
    w = np.exp(z - z.max())
    w = w / w.sum()
    return w @ V, w


def oracle_decode_row(cache, q_bits, table_row, L, ph, sigma):
    """One output row o[D] for one query head (bf16 bits q_bits[D])."""
    if L == 0:
        return np.zeros(cache.D)
    K, V = gather_unit(cache, table_row, ph, L)
    o, _ = attention_f64(bf16_to_f64(q_bits), K, V, sigma)
    return o


def oracle_decode(cache, q, block_table, lens, sigma, flags=None):
    """out[b][hq][:] in fp64 for q bf16 bits [B][Hq][D]."""
    B, Hq, D = q.shape
    G = Hq // cache.Hkv
    out = np.zeros((B, Hq, D))
    for (b, h, row, ph) in units(cache.layout, B, cache.Hkv):
        if flags is not None and flags[b] != 0:
            continue
        L = int(lens[row])
        if L == 0:
            continue
        K, V = gather_unit(cache, block_table[row], ph, L)
        for g in range(G):
            hq = h * G + g
            out[b, hq], _ = attention_f64(bf16_to_f64(q[b, hq]), K, V, sigma)
    return out


def oracle_decode_multi(cache, q, block_table, lens, sigma, flags=None):
    """R8: out[b][t][hq][:] in fp64 for q bf16 bits [B][T][Hq][D]."""
    B, T, Hq, D = q.shape
    G = Hq // cache.Hkv
    out = np.zeros((B, T, Hq, D))
    for (b, h, row, ph) in units(cache.layout, B, cache.Hkv):
        if flags is not None and flags[b] != 0:
            continue
        L = int(lens[row])
        if L <= 0:
            continue
        K, V = gather_unit(cache, block_table[row], ph, L)
        for t in range(T):
            n = L - T + t + 1            # tokens visible to draft t
            if n <= 0:
                continue
            for g in range(G):
                hq = h * G + g
                out[b, t, hq], _ = attention_f64(bf16_to_f64(q[b, t, hq]), K[:n], V[:n], sigma)
    return out


# ------------------------------------------------------ eviction scores
def oracle_attention_mass(cache, q, block_table, lens, sigma, flags=None):
    """R9: per unit, the step's attention mass on each of its L tokens.

    Returns {(b, h): fp64 [L]} = sum over the G query heads of the unit of the
    softmax weights (each head's weights sum to 1, so the masses sum to G).
    Flagged sequences and empty units are absent.
    """
    B, Hq, D = q.shape
    G = Hq // cache.Hkv
    mass = {}
    for (b, h, row, ph) in units(cache.layout, B, cache.Hkv):
        if flags is not None and flags[b] != 0:
            continue
        L = int(lens[row])
        if L <= 0:
            continue
        K, V = gather_unit(cache, block_table[row], ph, L)
        m = np.zeros(L)
        for g in range(G):
            _, wts = attention_f64(bf16_to_f64(q[b, h * G + g]), K, V, sigma)
            m += wts
        mass[(b, h)] = m
    return mass


def oracle_score_update(layout, scores, block_table, lens, mass, page_size):
    """Add the masses to the paged score array (fp32 [P][heads][S]) in place.

    The sum is taken in fp64 and rounded once to fp32 per slot.
    """
    for (b, h), m in mass.items():
        row = (b,) if layout == "seq" else (b, h)
        ph = h if layout == "seq" else 0
        for t in range(len(m)):
            pid = int(block_table[row][t // page_size])
            slot = t % page_size
            scores[pid, ph, slot] = np.float32(np.float64(scores[pid, ph, slot]) + m[t])
    return scores


# ------------------------------------------------------------ compaction
def oracle_compact(cache, block_table, lens, keep, n_keep, new_table, scores=None):
    """R10: rewrite each unit's kept tokens into the pages of new_table.

    keep: int32 [units][max_keep] strictly increasing positions (< L) of the
    tokens a unit keeps, n_keep [units] how many; units are in unit order
    (SEQ: (b, h) with b outer; HEAD: the same).  new_table has the old table's
    layout and never names a page the old table reads.  Returns the new
    cache (a copy) and the new scores (a copy) or None.
    """
    c = cache.copy()
    new_scores = None if scores is None else scores.copy()
    S, D = cache.S, cache.D
    B = block_table.shape[0]
    for i, (b, h, row, ph) in enumerate(units(cache.layout, B, cache.Hkv)):
        n = int(n_keep[i])
        pos = [int(x) for x in keep[i][:n]]
        for p0 in range(0, n, S):
            chunk = pos[p0:p0 + S]
            pid_new = int(new_table[row][p0 // S])
            src = [(int(block_table[row][t // S]), t % S) for t in chunk]
            slots = np.arange(len(chunk))
            for pool_old, pool_new, sc_old, sc_new in ((cache.k, c.k, cache.k_scale, c.k_scale),
                                                       (cache.v, c.v, cache.v_scale, c.v_scale)):
                if cache.kv_dtype == "bf16":
                    pool_new[pid_new, ph, slots] = [pool_old[p, ph, sl] for p, sl in src]
                    continue
                x = np.stack([(e4m3_to_f64(pool_old[p, ph, sl]).astype(np.float32)
                               * sc_old[p, ph]).astype(np.float32) for p, sl in src])
                amax = np.float32(np.max(np.abs(x)))
                s_new = np.float32(amax / E4M3_MAX_F32)
                pool_new[pid_new, ph, slots] = _quantise(x, s_new)
                sc_new[pid_new, ph] = s_new
            if scores is not None:
                for j, (p, sl) in enumerate(src):
                    new_scores[pid_new, ph, j] = scores[p, ph, sl]
    return c, new_scores


def lse_partial(q, K, V, sigma):
    """(m, l, o_unnormalised) of one token subset, natural-log domain, fp64."""
    z = float(sigma) * (K @ q)
    m = z.max()
    p = np.exp(z - m)
    return m, p.sum(), p @ V


def lse_merge(parts):
    """Merge (m, l, o) partials of disjoint token subsets into the softmax output."""
    M = max(m for m, _, _ in parts)
    Lsum = sum(l * np.exp(m - M) for m, l, _ in parts)
    O = sum(o * np.exp(m - M) for m, _, o in parts)
    return O / Lsum
