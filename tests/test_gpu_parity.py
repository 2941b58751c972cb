"""Parity of the HIP path (through the C ABI) with the CPU oracle, on a GPU.

Bit-exact: pool bytes (read back through the documented block layout), FP8
scales and flags.  Floating point: BF16 outputs of unflagged rows against the
fp64 oracle, max-abs <= 1e-2 and mean-abs <= 1e-3; flagged rows exactly +0.0.
"""
import os
import sys

import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.layout import pool_to_logical
from decode_attention_paged_pa_amd.workloads import make_workload, to_bf16_bits
from oracle import (
    OracleCache,
    bf16_from_f32_rne,
    bf16_to_f64,
    oracle_append,
    oracle_decode,
    oracle_validate,
)
from tests.oracle_fill import oracle_chunks, oracle_sequences_parallel

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def log(msg):
    print("[parity] " + msg, file=sys.stderr, flush=True)


def out_f64(out):
    return bf16_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16))


def flags_of(dw):
    return dw.flags.cpu().numpy().view(np.uint32)


def expected_flags(w, exp_tags=None, check_tags=True):
    exp = (w.expected_tags if exp_tags is None else exp_tags) if check_tags else None
    return oracle_validate(w.layout, w.P, w.S, w.block_table, w.lens, w.page_tags, exp, w.W)


def logical_pools(dw):
    """The device pools read back once, as logical [P][H][S][D] codes, and the scales."""
    w = dw.w
    torch.cuda.synchronize()
    out = {}
    for which in ("k", "v"):
        raw = (dw.cache.k if which == "k" else dw.cache.v).cpu().numpy()
        out[which] = pool_to_logical(raw, which, w.layout, w.kv_dtype, w.P, w.Hkv, w.D)
        del raw
    if w.kv_dtype == "fp8":
        out["k_scale"] = dw.cache.k_scale.cpu().numpy()
        out["v_scale"] = dw.cache.v_scale.cpu().numpy()
    return out


def compare_pools(dw, ora, seqs, logical=None):
    w = dw.w
    logical = logical_pools(dw) if logical is None else logical
    for which in ("k", "v"):
        for b in seqs:
            r = ora[b]
            got = logical[which][r["pages"]]
            want = r[which]
            bad = np.argwhere(got != want)
            assert bad.size == 0, "%s pool of sequence %d differs at %d places, first %s" % (
                which, b, len(bad), bad[:3].tolist())
    if w.kv_dtype == "fp8":
        ks = logical["k_scale"]
        vs = logical["v_scale"]
        for b in seqs:
            r = ora[b]
            assert np.array_equal(ks[r["pages"]].view(np.uint32), r["k_scale"].view(np.uint32)), b
            assert np.array_equal(vs[r["pages"]].view(np.uint32), r["v_scale"].view(np.uint32)), b


def compare_outputs(out, ora, seqs, flags, what=""):
    got = out_f64(out)
    errs = []
    for b in seqs:
        if flags is not None and flags[b] != 0:
            assert np.all(out[b].view(torch.int16).cpu().numpy() == 0), "flagged row %d not +0" % b
            continue
        errs.append(np.abs(got[b] - ora[b]["out"]))
    if errs:
        e = np.concatenate([x.ravel() for x in errs])
        log("%s max-abs %.3g mean-abs %.3g over %d values" % (what, e.max(), e.mean(), e.size))
        assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS, (e.max(), e.mean())
        assert np.all(np.isfinite(got[[b for b in seqs if flags is None or flags[b] == 0]]))


def run_full_case(w, partitions, pools=True, chunk=16):
    """Every sequence of a full-size workload against the oracle, the oracle run
    in chunks of `chunk` sequences (one per worker) to bound host memory: pool
    bytes and scales of every page, flags, and every output row at each
    partition count (each chunk meets the max-abs and mean-abs bars)."""
    log("full: workload %d (%s) B=%d T=%d layout=%s kv=%s P=%d" % (
        w.cfg_id, w.name, w.B, w.q_len, w.layout, w.kv_dtype, w.P))
    dw = build_device_workload(w, log=log)
    dw.step_append()
    outs = {}
    for p in partitions:
        outs[p] = dw.decode(check=True, num_partitions=p).clone()
        torch.cuda.synchronize()
        fl = flags_of(dw)
        assert np.array_equal(fl, expected_flags(w)), fl
    logical = logical_pools(dw) if pools else None
    seqs = list(range(w.B))
    for part in oracle_chunks(w, seqs, chunk):
        if pools:
            compare_pools(dw, part, list(part), logical)
        for p in partitions:
            compare_outputs(outs[p], part, list(part), fl,
                            "sequences %d..%d partitions=%d" % (min(part), max(part), p))
        log("checked sequences %d..%d" % (min(part), max(part)))
    return dw, outs


def run_case(w, seqs=None, partitions=(0,), check=True, pools=True, fill_seqs=None):
    log("workload %d (%s) B=%d layout=%s kv=%s P=%d lens[:6]=%s" % (
        w.cfg_id, w.name, w.B, w.layout, w.kv_dtype, w.P, w.lens.ravel()[:6].tolist()))
    dw = build_device_workload(w, seqs=fill_seqs, log=log)
    dw.step_append()
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    ora = oracle_sequences_parallel(w, seqs)
    if pools:
        compare_pools(dw, ora, seqs)
    outs = {}
    for p in partitions:
        out = dw.decode(check=check, num_partitions=p)
        torch.cuda.synchronize()
        fl = flags_of(dw) if check else None
        if check:
            want = expected_flags(w)
            assert np.array_equal(fl, want), (fl, want)
        compare_outputs(out, ora, seqs, fl, "partitions=%d" % p)
        outs[p] = out
    return dw, ora, outs


def test_workload1_tiny():
    w = make_workload(1)
    dw, ora, outs = run_case(w, partitions=(0, 1, 2, 32))
    assert pa.num_partitions(dw.cache, dw.block_table, dw.lens, w.Hq) == 1


def test_workload2_reduced_ragged_and_partition_counts():
    w = make_workload(2, batch=5, lens=[1, 17, 300, 1037, 4096])
    dw, ora, outs = run_case(w, partitions=(0, 1, 2, 3, 8, 64))
    # bitwise run-to-run determinism at a fixed partition count
    a = dw.decode(num_partitions=8)
    b = dw.decode(num_partitions=8)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_workload2_full():
    run_case(make_workload(2), partitions=(0, 8, 32))   # 32: a wave streams 2 partitions


def test_workload3_reduced_stale_tags():
    w = make_workload(3, batch=6, lens=[16, 17, 999, 4096, 5000, 16384], stale_frac=0.02)
    assert w.stale.any()
    run_case(w, partitions=(0, 4))


def test_workload3_full_stale_then_valid():
    w = make_workload(3)
    dw, ora, outs = run_case(w, partitions=(0, 16))       # 16: a wave streams 2 partitions
    fl = flags_of(dw)
    assert np.count_nonzero(fl) > 0
    # the same cache with every expected tag valid: all rows compared
    dw.expected_tags.copy_(dw.page_tags[dw.block_table.clamp(0, w.P - 1).long()].view(
        dw.expected_tags.shape))
    out = dw.decode(check=True)
    torch.cuda.synchronize()
    assert np.all(flags_of(dw) == 0)
    compare_outputs(out, ora, range(w.B), flags_of(dw), "all tags valid")


@pytest.mark.parametrize("layout,kv,D", [("head", "fp8", 128), ("head", "fp8", 64),
                                          ("head", "bf16", 64), ("seq", "fp8", 64)])
def test_cache_format_combinations(layout, kv, D):
    """Cache formats no named workload uses (the llama8b-bf16 shape with the format
    overridden), stale tags included: every layout x dtype x head size the C ABI takes."""
    if layout == "head":
        lens = np.array([[1, 17, 300, 1500, 4097, 16, 33, 900],
                         [2048, 5, 64, 65, 700, 4096, 1, 250]])
    else:
        lens = [1, 17, 300, 1500, 4097]
    w = make_workload(2, lens=lens, kv=kv, layout=layout, head_dim=D, stale_frac=0.02)
    run_case(w, partitions=(0, 1, 3))


@pytest.mark.parametrize("heads,layout,kv", [((8, 8), "seq", "fp8"), ((32, 32), "head", "bf16"),
                                              ((12, 6), "seq", "bf16"), ((12, 6), "head", "fp8")])
def test_group_sizes(heads, layout, kv):
    """G = 1 (as many query heads as KV heads, one valid column per MFMA tile) and
    Hkv = 6 (not a multiple of 4: the plain workgroup order), both layouts."""
    Hkv = heads[1]
    if layout == "head":
        rng = np.random.default_rng(Hkv)
        lens = rng.integers(1, 3000, size=(3, Hkv)).astype(np.int32)
    else:
        lens = [1, 700, 2900]
    w = make_workload(2, lens=lens, heads=heads, kv=kv, layout=layout, stale_frac=0.02)
    run_case(w, partitions=(0, 1, 4))


def test_workload4_headwise_full():
    run_case(make_workload(4), partitions=(0, 16, 64))


@pytest.mark.timeout(900)
def test_bf16_pools_beyond_4gib_sampled():
    """The 70B shape with a BF16 cache: each pool is 4.3 GB, so page offsets pass
    2^32 bytes (64-bit address arithmetic in append, validation and decode).  Two
    sampled sequences that hold pages past the 4 GiB mark are checked against
    the oracle; all rows are checked finite."""
    w = make_workload(5, kv="bf16", stale_frac=0.0)
    per_page = w.Hkv * w.S * w.D * 2
    far = [b for b in range(w.B)
           if (w.block_table[b][: -(-int(w.lens[b]) // w.S)].astype(np.int64) * per_page
               >= 1 << 32).any()]
    assert len(far) >= 2, far
    sampled = far[:2]
    dw, ora, outs = run_case(w, seqs=sampled, partitions=(0,), pools=False)
    got = out_f64(outs[0])
    assert np.all(np.isfinite(got))


def _custom_cache_case(K, V, q, S=16, kv="bf16"):
    """One sequence (Hkv = 1) with given K/V tokens, on GPU and in the oracle."""
    L, D = K.shape
    n_pages = -(-L // S)
    P = n_pages + 2
    rng = np.random.default_rng(L)
    bt = np.full((1, n_pages), 0x7FFFFFFF, np.int32)
    bt[0] = rng.permutation(P)[:n_pages]
    cache = pa.PagedKVCache("seq", kv, P, 1, D)
    btd = torch.from_numpy(bt).cuda()
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), L, dtype=torch.int32, device="cuda")
    kd = torch.from_numpy(K[None, None].copy()).view(torch.bfloat16).cuda()
    vd = torch.from_numpy(V[None, None].copy()).view(torch.bfloat16).cuda()
    pa.append(cache, btd, zero, n, kd, vd)
    qd = torch.from_numpy(q[None, None].copy()).view(torch.bfloat16).cuda()
    out = pa.decode(cache, qd, btd, n, np.float32(1 / np.sqrt(D)))
    oc = OracleCache("seq", kv, P, S, 1, D)
    oracle_append(oc, bt, np.zeros(1, np.int32), np.array([L], np.int32), K[None, None],
                  V[None, None], n_pages)
    ref = oracle_decode(oc, q[None, None], bt, np.array([L], np.int32), np.float32(1 / np.sqrt(D)))
    return out_f64(out)[0, 0], ref[0, 0]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_single_token_returns_v(kv):
    rng = np.random.default_rng(3)
    for D in (64, 128):
        K = to_bf16_bits(rng.standard_normal((1, D)).astype(np.float32))
        V = to_bf16_bits(rng.standard_normal((1, D)).astype(np.float32))
        q = to_bf16_bits(rng.standard_normal(D).astype(np.float32))
        got, ref = _custom_cache_case(K, V, q, kv=kv)
        want = bf16_to_f64(bf16_from_f32_rne(ref.astype(np.float32)))
        if kv == "bf16":
            assert np.array_equal(got, want)              # exactly V
        else:  # within one bf16 ulp of the rounded oracle
            ulp = 2.0 ** (np.floor(np.log2(np.abs(want) + 1e-30)) - 7)
            assert np.all(np.abs(got - want) <= ulp)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_identical_keys_give_mean_of_v(kv):
    rng = np.random.default_rng(4)
    L, D = 301, 128
    K = np.repeat(to_bf16_bits(rng.standard_normal((1, D)).astype(np.float32)), L, axis=0)
    V = to_bf16_bits(rng.standard_normal((L, D)).astype(np.float32))
    q = to_bf16_bits(rng.standard_normal(D).astype(np.float32))
    got, ref = _custom_cache_case(K, V, q, kv=kv)
    assert np.max(np.abs(got - ref)) <= MAX_ABS
    if kv == "bf16":
        assert np.max(np.abs(got - bf16_to_f64(V).mean(axis=0))) <= MAX_ABS


def test_large_score_range_rescaling():
    """Scores spread over a wide range force the running maximum to move often."""
    rng = np.random.default_rng(5)
    L, D = 2000, 128
    K = to_bf16_bits((rng.standard_normal((L, D)) * np.linspace(0.1, 8, L)[:, None]).astype(np.float32))
    V = to_bf16_bits(rng.standard_normal((L, D)).astype(np.float32))
    q = to_bf16_bits((rng.standard_normal(D) * 3).astype(np.float32))
    got, ref = _custom_cache_case(K, V, q)
    assert np.max(np.abs(got - ref)) <= MAX_ABS


def test_fault_injection_flags_and_zero_rows():
    w = make_workload(2, batch=6, lens=[40, 300, 700, 16, 5000, 1000], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    exp = w.expected_tags.copy()
    bt = w.block_table.copy()
    L = w.lens.copy()
    exp[1, 3] ^= 1                        # stale tag in sequence 1
    bt[2, 10] = w.P + 3                   # out-of-range id in sequence 2
    L[3] = w.W * 16 + 5                   # too long in sequence 3
    bt[4, 200] = -1                       # never read: sequence 4 has ceil(5000/16)=313 pages
    bt[4, 400] = -1                       # past its pages: not checked
    dw.expected_tags.copy_(torch.from_numpy(exp.view(np.int32)).cuda())
    dw.block_table.copy_(torch.from_numpy(bt).cuda())
    dw.lens.copy_(torch.from_numpy(L).cuda())
    out = dw.decode(check=True, num_partitions=4)
    torch.cuda.synchronize()
    want = oracle_validate(w.layout, w.P, w.S, bt, L, w.page_tags, exp, w.W)
    assert want.tolist() == [0, 1, 2, 6, 2, 0]   # sequence 3 also reads unused entries
    assert np.array_equal(flags_of(dw), want)
    o = out.view(torch.int16).cpu().numpy()
    for b in (1, 2, 3, 4):
        assert np.all(o[b] == 0)
    # range/length checks without a tag tracker
    out2 = pa.decode(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, expected_tags=None,
                     flags=dw.flags)
    torch.cuda.synchronize()
    want2 = oracle_validate(w.layout, w.P, w.S, bt, L, w.page_tags, None, w.W)
    assert np.array_equal(flags_of(dw), want2)
    assert torch.equal(out2[0].view(torch.int16), out[0].view(torch.int16))


def test_noop_tracker_matches_checked_run():
    w = make_workload(3, batch=4, lens=[100, 2000, 4097, 9000], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    a = dw.decode(check=True)
    b = dw.decode(check=False)
    torch.cuda.synchronize()
    assert np.all(flags_of(dw) == 0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_append_flags_and_out_of_range_pages_untouched():
    w = make_workload(2, batch=3, lens=[33, 64, 100], stale_frac=0.0)
    dw = build_device_workload(w)
    before = dw.cache.k.clone()
    bt = dw.block_table.clone()
    bt[1, 3] = w.P + 100                  # the step append of sequence 1 lands in page 3 (token 63)
    flags = torch.full((w.B,), -1, dtype=torch.int32, device="cuda")
    lens_old = dw.lens_old.clone()
    lens_old[2] = w.W * 16                # no room: length overflow
    pa.append(dw.cache, bt, lens_old, dw.n_step, dw.k_step, dw.v_step, flags=flags)
    torch.cuda.synchronize()
    assert flags.cpu().numpy().view(np.uint32).tolist() == [0, 2, 4]
    changed = (dw.cache.k != before).nonzero().numel()
    # only sequence 0's step token (one token x Hkv heads x D dims, 2 bytes each) changed at most
    assert changed <= w.Hkv * w.D * 2
