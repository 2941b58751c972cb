"""pa_decode_step (a decode step's append and decode in one call) on the GPU.

The step's append runs in the same launch as the decode's validation and split
plan, and writes only pages whose tag is the expected one.  Its pages, scales,
outputs and flags must be those of pa_cache_append (with the expected tags)
followed by pa_decode / pa_decode_multi, bit for bit; the outputs are also
checked against the fp64 oracle with the bars of the other parity tests
(max-abs 1e-2, mean-abs 1e-3, flags bit-exact, flagged rows +0.0).
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.layout import v_block_slots
from decode_attention_paged_pa_amd.workloads import make_workload
from tests.oracle_fill import oracle_sequences_parallel
from tests.test_gpu_parity import compare_outputs, compare_pools, expected_flags, flags_of, log

pytestmark = pytest.mark.gpu


def _state(cache):
    """The cache's bytes: pools, and FP8 scales as raw bits (NaN-safe)."""
    ts = [cache.k, cache.v] + [t for t in (cache.k_scale, cache.v_scale) if t is not None]
    return [t.contiguous().view(torch.uint8).clone() for t in ts]


def _restore(cache, snap):
    ts = [cache.k, cache.v] + [t for t in (cache.k_scale, cache.v_scale) if t is not None]
    for t, s in zip(ts, snap):
        t.view(torch.uint8).copy_(s)


@pytest.mark.parametrize("cfg,kw,parts", [
    (1, {}, 0),                                                        # BF16, D 64, one partition
    (3, dict(batch=4, lens=[100, 2000, 4097, 9000]), 4),               # FP8, stale tags, split-K 4
    (3, dict(batch=4, lens=[17, 33, 4096, 5000], stale_frac=0.0), 0),  # fresh pages, balanced split
    (4, dict(batch=2), 0),                                             # HEAD layout, ragged heads
    (2, dict(lens=np.array([[40, 1, 700, 16, 17, 3001, 0, 64], [5, 900, 33, 2000, 1, 48, 300, 15]]),
             kv="fp8", layout="head", stale_frac=0.02), 0),                       # HEAD FP8
    (2, dict(batch=3, lens=[40, 700, 3000], q_len=4), 0),              # 4 drafts
    (3, dict(batch=3, lens=[9, 300, 2049], q_len=8, stale_frac=0.0), 0),   # 8 drafts, FP8
])
def test_step_matches_append_then_decode(cfg, kw, parts):
    w = make_workload(cfg, **kw)
    log("step: workload %d B=%d layout=%s kv=%s T=%d parts=%d" % (
        cfg, w.B, w.layout, w.kv_dtype, w.q_len, parts))
    dw = build_device_workload(w)
    before = _state(dw.cache)
    dw.step_append()
    ref = dw.decode(check=True, num_partitions=parts).clone()
    torch.cuda.synchronize()
    ref_flags = dw.flags.clone()
    ref_state = _state(dw.cache)
    _restore(dw.cache, before)
    dw.flags.fill_(-1)
    out = dw.decode_step(check=True, num_partitions=parts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(dw.flags, ref_flags)
    for got, want in zip(_state(dw.cache), ref_state):
        assert torch.equal(got, want)


@pytest.mark.parametrize("cfg,kw", [
    (3, dict(batch=6, lens=[1, 16, 17, 500, 4097, 12000], stale_frac=0.0)),
    (3, dict(batch=5, lens=[20, 300, 700, 2000, 5000])),               # stale tags: flags
    (2, dict(batch=3, lens=[8, 900, 2500], q_len=4, kv="fp8")),
])
def test_step_against_oracle(cfg, kw):
    w = make_workload(cfg, **kw)
    log("step vs oracle: workload %d B=%d kv=%s T=%d" % (cfg, w.B, w.kv_dtype, w.q_len))
    dw = build_device_workload(w)
    out = dw.decode_step(check=True)
    torch.cuda.synchronize()
    fl = flags_of(dw)
    assert np.array_equal(fl, expected_flags(w)), fl
    seqs = list(range(w.B))
    ora = oracle_sequences_parallel(w, seqs)
    compare_pools(dw, ora, seqs)
    compare_outputs(out, ora, seqs, fl, "step")


def test_step_without_new_tokens_is_the_decode():
    w = make_workload(2, batch=3, lens=[50, 600, 1500], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    ref = dw.decode(check=True).clone()
    before = _state(dw.cache)
    zero = torch.zeros_like(dw.n_step)
    k0 = dw.k_step[:, :, :0].contiguous()
    out = pa.decode_step(dw.cache, dw.q, dw.block_table, dw.lens, zero, k0, k0, dw.lens, w.sigma,
                         expected_tags=dw.expected_tags, flags=dw.flags)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    for got, want in zip(_state(dw.cache), before):
        assert torch.equal(got, want)


@pytest.mark.parametrize("kv,layout", [("fp8", "seq"), ("bf16", "seq"), ("fp8", "head")])
def test_step_append_through_a_stale_entry_leaves_the_page_alone(kv, layout):
    """Sequence 1's step token lands in table entry i, which is stale: it names
    page X, now a full page of sequence 0 (whose tag moved on).  The step must
    leave X's bytes and scales alone, flag sequence 1 only, and give sequence 0
    its oracle output; pa_cache_append with the expected tags does the same and
    flags the page (the integrity-check paragraph: the check protects requests
    that share GPU memory)."""
    if layout == "head":
        lens = np.array([[700, 300, 33, 900, 64, 17, 450, 1000], [500, 81, 600, 20, 90, 700, 3, 40]])
    else:
        lens = [700, 501]
    w = make_workload(3, lens=lens, kv=kv, layout=layout, stale_frac=0.0)
    dw = build_device_workload(w)
    row1 = (1,) if layout == "seq" else (1, 0)
    row0 = (0,) if layout == "seq" else (0, 0)
    L1 = int(w.lens[row1])
    i = (L1 - 1) // 16                                 # the entry holding sequence 1's step token
    X = int(w.block_table[row0][5])                    # a full page of sequence 0
    bt = w.block_table.copy()
    exp = w.expected_tags.copy()
    bt[row1][i] = X
    exp[row1][i] = np.uint32((int(w.page_tags[X]) - 1) % 2 ** 32)
    dw.block_table.copy_(torch.from_numpy(bt).cuda())
    dw.expected_tags.copy_(torch.from_numpy(exp.view(np.int32)).cuda())
    before = _state(dw.cache)
    out = dw.decode_step(check=True)
    torch.cuda.synchronize()
    assert flags_of(dw).tolist() == [0, 1]
    after = _state(dw.cache)
    kp_b, kp_a = before[0].view(w.P, -1), after[0].view(w.P, -1)
    changed = set((kp_a != kp_b).any(dim=1).nonzero().flatten().tolist())
    # the step pages of every unit but the stale one (HEAD: sequence 1's other
    # heads append into their own pages)
    units = [(0,), (1,)] if layout == "seq" else [(b, h) for b in range(2) for h in range(w.Hkv)]
    steps = {int(w.block_table[u][(int(w.lens[u]) - 1) // 16]) for u in units if u != row1}
    assert changed <= steps, (changed, steps)
    assert X not in changed
    sp, sh = v_block_slots(w.layout, w.P, w.Hkv)      # X's V blocks sit in other slots
    H = w.Hkv if layout == "seq" else 1
    vp_b, vp_a = before[1].view(w.P, H, -1), after[1].view(w.P, H, -1)
    for h in range(H):
        assert torch.equal(vp_a[sp[X, h], sh[X, h]], vp_b[sp[X, h], sh[X, h]])
    if kv == "fp8":
        for j in (2, 3):
            assert torch.equal(after[j].view(w.P, -1)[X], before[j].view(w.P, -1)[X])
    w2 = make_workload(3, lens=lens, kv=kv, layout=layout, stale_frac=0.0)
    w2.block_table, w2.expected_tags = bt, exp
    ora = oracle_sequences_parallel(w2, [0])
    compare_outputs(out, ora, [0, 1], flags_of(dw), "stale entry")
    # the same through pa_cache_append: the page is left alone and flagged
    _restore(dw.cache, before)
    fl = torch.full((w.B,), -1, dtype=torch.int32, device="cuda")
    pa.append(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step, dw.v_step, flags=fl,
              expected_tags=dw.expected_tags)
    torch.cuda.synchronize()
    assert fl.cpu().numpy().view(np.uint32).tolist() == [0, 1]
    assert torch.equal(_state(dw.cache)[0].view(w.P, -1)[X], kp_b[X])
