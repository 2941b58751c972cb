"""C-ABI checks that need no GPU: the library loads, exports every function that
include/pa.h declares, and rejects bad arguments before any launch.

Device pointers here are fake (aligned, never dereferenced): every call below
must fail its argument checks and return before touching the GPU.
"""
import ctypes
import os
import re

import pytest

from decode_attention_paged_pa_amd import pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000  # 256-byte aligned stand-in for a device pointer

pytestmark = pytest.mark.skipif(not os.path.exists(pa.LIB_PATH), reason="libpa.so not built")


def _declared_functions():
    """Every pa_* function that a header under include/ declares."""
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("pa_cache_append", "pa_decode", "pa_decode_workspace_bytes", "pa_strerror",
              "pa_decode_multi", "pa_decode_multi_workspace_bytes", "pa_decode_scored",
              "pa_cache_compact", "pa_prefill", "pa_prefill_workspace_bytes", "pa_decode_step"):
        assert n in names


def test_library_exports_every_declared_function():
    L = pa.lib()
    names = _declared_functions()
    assert "pa_probe_stream" in names and "pa_probe_gather" in names
    for n in names:
        assert hasattr(L, n), n


def test_probe_argument_errors():
    """The read-ceiling probes refuse bad shapes before any launch."""
    L = pa.lib()
    vp = ctypes.c_void_p
    E = -1   # PA_ERR_INVALID_ARG
    assert L.pa_probe_stream(None, 1 << 20, 64, vp(FAKE), None) == E
    assert L.pa_probe_stream(vp(FAKE + 4), 1 << 20, 64, vp(FAKE), None) == E     # misaligned
    assert L.pa_probe_stream(vp(FAKE), 1 << 20, 62, vp(FAKE), None) == E         # waves % 4
    assert L.pa_probe_stream(vp(FAKE), (1 << 20) + 512, 64, vp(FAKE), None) == E  # bytes % (1 KiB * waves)
    ok = dict(pool=vp(FAKE), pool_bytes=1 << 24, ids=vp(FAKE), waves=64, ipw=16, bb=2048,
              inf=2, sink=vp(FAKE))

    def g(**kw):
        a = dict(ok, **kw)
        return L.pa_probe_gather(a["pool"], a["pool_bytes"], a["ids"], a["waves"], a["ipw"],
                                 a["bb"], a["inf"], a["sink"], None)
    assert g(bb=3000) == E
    assert g(inf=3) == E
    assert g(ipw=6, inf=4) == E
    assert g(pool_bytes=1024) == E
    assert g(ids=None) == E
    assert g(waves=0) == E


def _cache(**kw):
    d = dict(layout=0, kv_dtype=0, num_pages=100, page_size=16, num_kv_heads=8, head_dim=128,
             k_pages=FAKE, v_pages=FAKE + (1 << 20), k_scale=None, v_scale=None, page_tags=None)
    d.update(kw)
    return pa.CacheDesc(**d)


def _seq(**kw):
    d = dict(batch=4, table_width=64, block_table=FAKE, lens=FAKE + 4096, expected_tags=None)
    d.update(kw)
    return pa.SeqDesc(**d)


def _decode(cache, seq, hq=32, q=FAKE, out=FAKE, scale=0.088, parts=0, flags=None, ws=None,
            ws_bytes=0):
    L = pa.lib()
    return L.pa_decode(ctypes.byref(cache), ctypes.byref(seq), hq, ctypes.c_void_p(q),
                       ctypes.c_void_p(out), scale, parts,
                       ctypes.c_void_p(flags) if flags else None,
                       ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_pool_bytes_and_the_fp8_halving():
    """FP8 halves the pool ("Cloudflare quantizes Kimi and GLM caches", KV cache
    quantization paragraph: context held goes from about 686K to 1.37M tokens)."""
    import json

    facts = json.load(open(os.path.join(ROOT, "tests", "golden", "page_size_facts.json")))
    f = facts["fp8_vs_bf16_context_tokens"]
    ratio = f["fp8_tokens"] / f["bf16_tokens"]
    L = pa.lib()
    bf = L.pa_pool_bytes(ctypes.byref(_cache(kv_dtype=0)))
    f8 = L.pa_pool_bytes(ctypes.byref(_cache(kv_dtype=1)))
    assert bf == 100 * 8 * 16 * 128 * 2
    assert abs(bf / f8 - ratio) < 0.01
    assert L.pa_pool_bytes(ctypes.byref(_cache(layout=1))) == 100 * 16 * 128 * 2
    assert L.pa_pool_bytes(ctypes.byref(_cache(kv_dtype=7))) == 0


def test_no_paging_window_matches_the_four_prompt_figure():
    """128K tokens of Llama-3.1-8B BF16 KV per prompt: four fit beside the weights
    on an 80 GB H100 ("How we built the most efficient inference engine",
    section "Batching to feed the Tensor Cores")."""
    import json

    f = json.load(open(os.path.join(ROOT, "tests", "golden", "page_size_facts.json")))
    f = f["no_paging_128k_prompts_h100"]
    c = _cache(num_pages=f["window_tokens"] // 16, num_kv_heads=f["llama31_8b_kv_heads"],
               head_dim=f["llama31_8b_head_dim"])
    per_layer = 2 * pa.lib().pa_pool_bytes(ctypes.byref(c))        # K and V
    per_prompt = per_layer * f["llama31_8b_layers"]
    assert per_prompt == 2 ** 34                                   # 16 GiB per 128K prompt
    assert round((f["h100_hbm_bytes"] - f["weights_bytes"]) / per_prompt) == f["prompts"]


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=32), -2), (dict(head_dim=96), -2), (dict(layout=5), -1),
    (dict(kv_dtype=3), -1), (dict(num_pages=0), -1), (dict(k_pages=None), -1),
    (dict(k_pages=FAKE + 8), -1), (dict(kv_dtype=1), -1),  # FP8 without scales
    (dict(num_kv_heads=1 << 19), -2),   # a SEQ page row of 2^31 bytes: page strides are 32-bit
])
def test_decode_rejects_bad_cache(kw, code):
    assert _decode(_cache(**kw), _seq()) == code


def test_decode_rejects_bad_arguments():
    c, s = _cache(), _seq()
    assert _decode(c, s, hq=30) == -1                      # Hq not a multiple of Hkv
    assert _decode(c, s, hq=8 * 17) == -2                  # group of 17 > 16
    assert _decode(c, s, q=0) == -1
    assert _decode(c, s, out=FAKE + 2) == -1               # misaligned output
    assert _decode(c, s, scale=float("nan")) == -1
    assert _decode(c, s, parts=-1) == -1
    assert _decode(c, _seq(batch=0)) == -1
    assert _decode(c, _seq(table_width=0)) == -1
    assert _decode(c, _seq(lens=None)) == -1
    # a tag check needs flags and page tags
    assert _decode(c, _seq(expected_tags=FAKE)) == -1
    # more than one partition needs a workspace of the advertised size
    L = pa.lib()
    need = L.pa_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, 4)
    assert need == 4 * 32 * 4 * (128 * 4) + 4 * 32 * 4 * 2 * 4
    assert _decode(c, s, parts=4) == -3
    assert _decode(c, s, parts=4, ws=FAKE, ws_bytes=need - 1) == -3
    assert _decode(c, s, parts=4, ws=FAKE + 16, ws_bytes=need) == -3


def test_partition_choice():
    L = pa.lib()
    c = _cache()
    n = lambda s, p: L.pa_decode_num_partitions(ctypes.byref(c), ctypes.byref(s), 64, p)  # noqa: E731
    assert n(_seq(batch=64, table_width=2048), 8) == 8
    assert n(_seq(batch=64, table_width=2048), 0) == 0     # auto: balanced at run time
    assert n(_seq(batch=4, table_width=32), 0) == 1        # tiny: one partition, no reduce
    assert n(_seq(batch=4, table_width=32), 3) == 3
    assert L.pa_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(_seq(table_width=32)), 64, 1) == 0
    assert L.pa_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(_seq(table_width=32)), 64, 0) == 0
    # balanced split: at most ceil(2048 / heads per pair) + groups pairs; per pair and head
    # G * T columns of D floats and (max, sum); then the plan (groups + 3 ints) and the
    # group of each pair, every block 256-byte aligned
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    ws = lambda cc, ss, hq=64: L.pa_decode_workspace_bytes(ctypes.byref(cc), ctypes.byref(ss), hq, 0)  # noqa: E731
    pairs = 2048 // 8 + 64                                  # SEQ: a pair holds the 8 heads of a sequence
    slots = pairs * 8 * 8
    assert ws(c, _seq(batch=64, table_width=2048)) == (
        a256(slots * 128 * 4) + a256(slots * 8) + a256((64 + 3) * 4) + a256(pairs * 4)
        + a256(pairs * 16))                                 # a record per pair slot
    ch = _cache(layout=1)                                   # HEAD: a pair is one unit's partition
    pairs = 2048 + 16 * 8
    slots = pairs * 4
    assert ws(ch, _seq(batch=16, table_width=2048), hq=32) == (
        a256(slots * 128 * 4) + a256(slots * 8) + a256((16 * 8 + 3) * 4) + a256(pairs * 4)
        + a256(pairs * 16) + a256(16 * 8 * 4))              # HEAD: one validation word per unit


def _decode_multi(cache, seq, hq=32, q_len=4, q=FAKE, out=FAKE, scale=0.088, parts=0, flags=None,
                  ws=None, ws_bytes=0):
    L = pa.lib()
    return L.pa_decode_multi(ctypes.byref(cache), ctypes.byref(seq), hq, q_len, ctypes.c_void_p(q),
                             ctypes.c_void_p(out), scale, parts,
                             ctypes.c_void_p(flags) if flags else None,
                             ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_decode_multi_rejects_bad_arguments():
    c, s = _cache(), _seq()
    assert _decode_multi(c, s, q_len=0) == -1
    assert _decode_multi(c, s, q_len=9) == -2              # more than 8 drafts
    assert _decode_multi(c, s, hq=8 * 16, q_len=8) == -2   # 16 heads x 8 tokens > 64 columns
    assert _decode_multi(c, s, hq=8 * 16, q_len=1, parts=4) == -3   # q_len 1: decode's limits
    assert _decode_multi(c, s, q=FAKE + 8) == -1
    assert _decode_multi(_cache(head_dim=96), s) == -2
    assert _decode_multi(c, _seq(expected_tags=FAKE)) == -1
    L = pa.lib()
    wsm = lambda hq, t, p: L.pa_decode_multi_workspace_bytes(  # noqa: E731
        ctypes.byref(c), ctypes.byref(s), hq, t, p)
    # partials of every (sequence, token, head, partition): D floats + (max, sum)
    assert wsm(32, 4, 4) == 4 * 4 * 32 * 4 * 128 * 4 + 4 * 4 * 32 * 4 * 2 * 4
    assert wsm(32, 1, 4) == L.pa_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, 4)
    assert wsm(64, 8, 1) == 0
    assert wsm(8 * 16, 8, 2) == ctypes.c_size_t(-1).value
    need = wsm(32, 4, 4)
    assert _decode_multi(c, s, parts=4, ws=FAKE, ws_bytes=need - 1) == -3


def test_decode_scored_arguments_and_workspace():
    L = pa.lib()
    c, s = _cache(), _seq()
    sc = lambda scores=FAKE, ws=None, ws_bytes=0, parts=0, hq=32: L.pa_decode_scored(  # noqa: E731
        ctypes.byref(c), ctypes.byref(s), hq, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 0.088,
        parts, None, ctypes.c_void_p(scores) if scores else None,
        ctypes.c_void_p(ws) if ws else None, ws_bytes, None)
    assert sc(scores=0) == -1
    assert sc(scores=FAKE + 2) == -1
    need1 = L.pa_decode_scored_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, 1)
    # the rows' final (max, sum) [B][Hq][2] fp32 (no partials at Pn = 1), then the score
    # pass's plan: (groups + 3) int32 and its pairs' groups, at most
    # max(ceil(4096 / Hkv) + groups, groups * ceil(W / 128)) pairs (SEQ: groups = B = 4)
    a256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    pairs = max(4096 // 8 + 4, 4 * 1)
    assert need1 == a256(4 * 32 * 2 * 4) + a256((4 + 3) * 4) + a256(pairs * 4)
    need4 = L.pa_decode_scored_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, 4)
    assert need4 == need1 + L.pa_decode_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, 4)
    assert sc(ws=None) == -3                                  # always needs a workspace
    assert sc(ws=FAKE, ws_bytes=need1 - 1, parts=1) == -3
    assert sc(hq=8 * 17) == -2


def test_compact_rejects_bad_arguments():
    L = pa.lib()
    c, s = _cache(), _seq()
    cp = lambda keep=FAKE, stride=16, n_keep=FAKE, nt=FAKE, scores=None, fl=None, cc=c: (  # noqa: E731
        L.pa_cache_compact(ctypes.byref(cc), ctypes.byref(s), ctypes.c_void_p(keep) if keep else None,
                           stride, ctypes.c_void_p(n_keep) if n_keep else None,
                           ctypes.c_void_p(nt) if nt else None,
                           ctypes.c_void_p(scores) if scores else None,
                           ctypes.c_void_p(fl) if fl else None, None))
    assert cp(keep=0) == -1
    assert cp(stride=0) == -1
    assert cp(n_keep=0) == -1
    assert cp(nt=0) == -1
    assert cp(keep=FAKE + 2) == -1
    assert cp(scores=FAKE + 1) == -1
    assert cp(fl=FAKE + 2) == -1
    assert cp(cc=_cache(head_dim=80)) == -2


def test_prefill_arguments_and_partitions():
    L = pa.lib()
    c = _cache()
    s = _seq(batch=4, table_width=2048)
    pf = lambda hq=32, cl=2048, parts=0, ws=None, ws_bytes=0: L.pa_prefill(  # noqa: E731
        ctypes.byref(c), ctypes.byref(s), hq, cl, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
        0.088, parts, None, ctypes.c_void_p(ws) if ws else None, ws_bytes, None)
    assert pf(cl=0) == -1
    assert pf(cl=2048 * 16 + 1) == -1                     # longer than the table holds
    assert pf(hq=8 * 17) == -2
    n = lambda cl, p: L.pa_prefill_num_partitions(ctypes.byref(c), ctypes.byref(s), 32, cl, p)  # noqa: E731
    # page-sharing prefill: 4 x 8 units x (4 heads x 2048 tokens / 32 / 4) workgroups of
    # four 32-column blocks = 2048 workgroups, above the 1536 aimed at: no split; a
    # 512-token chunk gives 512 workgroups: 3 partitions
    assert n(2048, 0) == 1
    assert n(512, 0) == 3
    # a short chunk gives few waves (32): the prefix is split into 64 partitions
    # of 32 pages (about 2048 waves, partitions no shorter than 32 pages)
    assert n(16, 0) == 64
    assert n(2048, 3) == 3
    wsb = lambda cl, p: L.pa_prefill_workspace_bytes(ctypes.byref(c), ctypes.byref(s), 32, cl, p)  # noqa: E731
    assert wsb(2048, 1) == 0
    assert wsb(64, 2) == 4 * 64 * 32 * 2 * 128 * 4 + 4 * 64 * 32 * 2 * 2 * 4
    assert pf(parts=2, cl=64, ws=FAKE, ws_bytes=wsb(64, 2) - 1) == -3


def test_append_rejects_bad_arguments():
    L = pa.lib()
    c, s = _cache(), _seq()
    ap = lambda cc, ss, n_new=FAKE, n_max=4, k=FAKE, v=FAKE, fl=None: L.pa_cache_append(  # noqa: E731
        ctypes.byref(cc), ctypes.byref(ss), ctypes.c_void_p(n_new) if n_new else None, n_max,
        ctypes.c_void_p(k) if k else None, ctypes.c_void_p(v) if v else None,
        ctypes.c_void_p(fl) if fl else None, None)
    assert ap(c, s, n_new=0) == -1
    assert ap(c, s, n_max=-1) == -1
    assert ap(c, s, k=0) == -1
    assert ap(c, s, v=FAKE + 1) == -1
    assert ap(_cache(head_dim=80), s) == -2
    assert ap(c, _seq(block_table=None)) == -1
    assert ap(c, s, n_max=0) == 0        # nothing to do, nothing launched


def test_decode_step_rejects_bad_arguments():
    L = pa.lib()
    c, s = _cache(), _seq()
    vp = lambda x: ctypes.c_void_p(x) if x else None  # noqa: E731

    def st(cc=c, ss=s, lens_old=FAKE + 8192, n_new=FAKE + 12288, n_max=1, k=FAKE, v=FAKE,
           hq=32, q_len=1, q=FAKE, out=FAKE, scale=0.088, parts=0, flags=None):
        return L.pa_decode_step(ctypes.byref(cc), ctypes.byref(ss), vp(lens_old), vp(n_new),
                                n_max, vp(k), vp(v), hq, q_len, vp(q), vp(out), scale, parts,
                                vp(flags), None, 0, None)
    assert st(lens_old=0) == -1
    assert st(lens_old=FAKE + 2) == -1                      # misaligned lengths
    assert st(n_new=0) == -1
    assert st(n_max=-1) == -1
    assert st(k=0) == -1                                   # tokens to append need k_new
    assert st(v=FAKE + 1) == -1
    assert st(hq=30) == -1                                 # then the decode's own checks
    assert st(q_len=9) == -2
    assert st(scale=float("nan")) == -1
    assert st(parts=4) == -3                               # its workspace, as pa_decode's
    assert st(cc=_cache(head_dim=80)) == -2
    assert st(ss=_seq(block_table=None)) == -1
    assert st(ss=_seq(expected_tags=FAKE)) == -1          # a tag check needs flags


def test_strerror_and_version():
    L = pa.lib()
    assert b"workspace" in L.pa_strerror(-3)
    assert L.pa_strerror(12345) == b"unknown error code"
    assert pa.version() >= 100
