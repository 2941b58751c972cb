"""Python binding of libpa (ctypes): argument marshalling only.

Every step of the decode path runs in the HIP kernels of libpa.so; this module
checks tensor dtypes, shapes and devices, passes raw device pointers and the
current HIP stream, and turns negative return codes into exceptions.  It has
no CPU fallback: without the built library every call raises.

Entry points mirror include/pa.h: append (pa_cache_append); decode
(pa_decode / pa_decode_timed), workspace_bytes, num_partitions; decode_multi
(pa_decode_multi: causal drafts), multi_workspace_bytes; decode_step
(pa_decode_step: append + decode in one call); decode_scored
(pa_decode_scored: eviction scores), scored_workspace_bytes; compact
(pa_cache_compact); prefill (pa_prefill), prefill_workspace_bytes,
prefill_num_partitions; version.  PagedKVCache owns the pools, scales and tags
(sized by pa_pool_bytes); DecodeStepGraph captures a step (decode_step, or
append + prefill) as one HIP graph.
"""
import ctypes
import os

import torch

# PA_LIB_PATH points the binding at another build of the library (an
# instrumented host build in the tests); by default, the in-tree libpa.so.
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "lib", "libpa.so")

LAYOUT = {"seq": 0, "head": 1}
KV_DTYPE = {"bf16": 0, "fp8": 1}
PAGE_SIZE = 16

PA_FLAG_TAG_MISMATCH = 1
PA_FLAG_PAGE_OOB = 2
PA_FLAG_LEN_OVERFLOW = 4


class PAError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s failed: %s (%d)" % (what, _strerror(code), code))
        self.code = code


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32), ("kv_dtype", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("page_tags", ctypes.c_void_p),
    ]


class SeqDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("table_width", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("lens", ctypes.c_void_p),
        ("expected_tags", ctypes.c_void_p),
    ]


_LIB = None


def lib():
    """The loaded libpa.so (torch's HIP runtime is loaded first so both share it)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libpa.so is not built (%s); run "
                               "`python -m decode_attention_paged_pa_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.pa_pool_bytes.argtypes = [P(CacheDesc)]
        L.pa_pool_bytes.restype = sz
        L.pa_cache_append.argtypes = [P(CacheDesc), P(SeqDesc), vp, i32, vp, vp, vp, vp]
        L.pa_cache_append.restype = ctypes.c_int
        L.pa_decode_workspace_bytes.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32]
        L.pa_decode_workspace_bytes.restype = sz
        L.pa_decode_num_partitions.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32]
        L.pa_decode_num_partitions.restype = ctypes.c_int
        L.pa_decode.argtypes = [P(CacheDesc), P(SeqDesc), i32, vp, vp, ctypes.c_float, i32, vp,
                                vp, sz, vp]
        L.pa_decode.restype = ctypes.c_int
        L.pa_decode_timed.argtypes = [P(CacheDesc), P(SeqDesc), i32, vp, vp, ctypes.c_float, i32,
                                      vp, vp, sz, vp, P(vp)]
        L.pa_decode_timed.restype = ctypes.c_int
        L.pa_decode_multi.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, vp, vp, ctypes.c_float,
                                      i32, vp, vp, sz, vp]
        L.pa_decode_multi.restype = ctypes.c_int
        L.pa_decode_multi_timed.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, vp, vp,
                                            ctypes.c_float, i32, vp, vp, sz, vp, P(vp)]
        L.pa_decode_multi_timed.restype = ctypes.c_int
        L.pa_decode_multi_workspace_bytes.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, i32]
        L.pa_decode_multi_workspace_bytes.restype = sz
        L.pa_decode_scored.argtypes = [P(CacheDesc), P(SeqDesc), i32, vp, vp, ctypes.c_float, i32,
                                       vp, vp, vp, sz, vp]
        L.pa_decode_scored.restype = ctypes.c_int
        L.pa_decode_scored_timed.argtypes = [P(CacheDesc), P(SeqDesc), i32, vp, vp, ctypes.c_float,
                                             i32, vp, vp, vp, sz, vp, P(vp)]
        L.pa_decode_scored_timed.restype = ctypes.c_int
        L.pa_decode_scored_workspace_bytes.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32]
        L.pa_decode_scored_workspace_bytes.restype = sz
        L.pa_cache_compact.argtypes = [P(CacheDesc), P(SeqDesc), vp, i32, vp, vp, vp, vp, vp]
        L.pa_cache_compact.restype = ctypes.c_int
        L.pa_decode_step.argtypes = [P(CacheDesc), P(SeqDesc), vp, vp, i32, vp, vp, i32, i32, vp,
                                     vp, ctypes.c_float, i32, vp, vp, sz, vp]
        L.pa_decode_step.restype = ctypes.c_int
        L.pa_decode_step_timed.argtypes = [P(CacheDesc), P(SeqDesc), vp, vp, i32, vp, vp, i32,
                                           i32, vp, vp, ctypes.c_float, i32, vp, vp, sz, vp,
                                           P(vp)]
        L.pa_decode_step_timed.restype = ctypes.c_int
        L.pa_prefill.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, vp, vp, ctypes.c_float, i32,
                                 vp, vp, sz, vp]
        L.pa_prefill.restype = ctypes.c_int
        L.pa_prefill_timed.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, vp, vp, ctypes.c_float,
                                       i32, vp, vp, sz, vp, P(vp)]
        L.pa_prefill_timed.restype = ctypes.c_int
        L.pa_prefill_workspace_bytes.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, i32]
        L.pa_prefill_workspace_bytes.restype = sz
        L.pa_prefill_num_partitions.argtypes = [P(CacheDesc), P(SeqDesc), i32, i32, i32]
        L.pa_prefill_num_partitions.restype = ctypes.c_int
        L.pa_strerror.argtypes = [ctypes.c_int]
        L.pa_strerror.restype = ctypes.c_char_p
        L.pa_version.argtypes = []
        L.pa_version.restype = ctypes.c_int
        L.pa_decode_noalloc.argtypes = [P(CacheDesc), P(SeqDesc), i32, vp, vp, ctypes.c_float,
                                        i32, vp, vp]
        L.pa_decode_noalloc.restype = ctypes.c_int
        L.pa_probe_stream.argtypes = [vp, sz, i32, vp, vp]
        L.pa_probe_stream.restype = ctypes.c_int
        L.pa_probe_gather.argtypes = [vp, sz, vp, i32, i32, i32, i32, vp, vp]
        L.pa_probe_gather.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _strerror(code):
    try:
        return lib().pa_strerror(code).decode()
    except Exception:  # library missing: still report the code
        return "error"


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtypes, device=True):
    if t is None:
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if device and t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


I32 = (torch.int32,)
U32 = (torch.int32, torch.uint32)
BF16 = (torch.bfloat16, torch.int16, torch.uint16)


class PagedKVCache:
    """The physical cache: K/V pools (raw bytes), FP8 scales and page tags.

    Pools are allocated with the byte size pa_pool_bytes reports and filled with
    NaN patterns (0x7FC0 for BF16, 0x7F for FP8) so that a read of an unwritten
    slot shows up in the results.
    """

    def __init__(self, layout, kv_dtype, num_pages, num_kv_heads, head_dim, device="cuda",
                 page_tags=None, poison=True):
        self.layout, self.kv_dtype = layout, kv_dtype
        self.num_pages, self.num_kv_heads, self.head_dim = int(num_pages), int(num_kv_heads), int(head_dim)
        self.page_size = PAGE_SIZE
        d = CacheDesc(LAYOUT[layout], KV_DTYPE[kv_dtype], self.num_pages, PAGE_SIZE,
                      self.num_kv_heads, self.head_dim, None, None, None, None, None)
        nbytes = lib().pa_pool_bytes(ctypes.byref(d))
        if nbytes == 0:
            raise ValueError("invalid cache shape")
        self.pool_bytes = nbytes
        self.k = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.v = torch.empty(nbytes, dtype=torch.uint8, device=device)
        heads = self.num_kv_heads if layout == "seq" else 1
        if kv_dtype == "fp8":
            self.k_scale = torch.full((self.num_pages, heads), float("nan"), dtype=torch.float32, device=device)
            self.v_scale = torch.full_like(self.k_scale, float("nan"))
        else:
            self.k_scale = self.v_scale = None
        if poison:
            if kv_dtype == "bf16":
                self.k.view(torch.int16).fill_(0x7FC0)
                self.v.view(torch.int16).fill_(0x7FC0)
            else:
                self.k.fill_(0x7F)
                self.v.fill_(0x7F)
        self.page_tags = None if page_tags is None else _need(page_tags, "page_tags", U32)

    def new_scores(self):
        """Zeroed eviction scores, fp32 [P][Hkv (SEQ) or 1 (HEAD)][S], laid out like the pages."""
        heads = self.num_kv_heads if self.layout == "seq" else 1
        return torch.zeros((self.num_pages, heads, PAGE_SIZE), dtype=torch.float32,
                           device=self.k.device)

    def desc(self):
        return CacheDesc(LAYOUT[self.layout], KV_DTYPE[self.kv_dtype], self.num_pages, PAGE_SIZE,
                         self.num_kv_heads, self.head_dim, _ptr(self.k), _ptr(self.v),
                         _ptr(self.k_scale), _ptr(self.v_scale), _ptr(self.page_tags))


def _seq(cache, block_table, lens, expected_tags=None):
    _need(block_table, "block_table", I32)
    _need(lens, "lens", I32)
    if cache.layout == "seq":
        if block_table.dim() != 2 or lens.dim() != 1 or lens.shape[0] != block_table.shape[0]:
            raise ValueError("SEQ layout expects block_table [B][W] and lens [B]")
    else:
        if (block_table.dim() != 3 or block_table.shape[1] != cache.num_kv_heads
                or tuple(lens.shape) != tuple(block_table.shape[:2])):
            raise ValueError("HEAD layout expects block_table [B][Hkv][W] and lens [B][Hkv]")
    if expected_tags is not None:
        _need(expected_tags, "expected_tags", U32)
        if tuple(expected_tags.shape) != tuple(block_table.shape):
            raise ValueError("expected_tags must have the block table's shape")
    return SeqDesc(block_table.shape[0], block_table.shape[-1], _ptr(block_table), _ptr(lens),
                   _ptr(expected_tags))


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def append(cache, block_table, lens, n_new, k_new, v_new, flags=None, stream=None,
           expected_tags=None):
    """pa_cache_append: write n_new[u] tokens of k_new/v_new [B][Hkv][n_max][D] (BF16);
    with expected_tags, only into pages whose tag is the expected one."""
    sd = _seq(cache, block_table, lens, expected_tags)
    _need(n_new, "n_new", I32)
    if tuple(n_new.shape) != tuple(lens.shape):
        raise ValueError("n_new must have the shape of lens")
    _need(k_new, "k_new", BF16)
    _need(v_new, "v_new", BF16)
    B = block_table.shape[0]
    if (k_new.dim() != 4 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.shape[0] != B
            or k_new.shape[1] != cache.num_kv_heads or k_new.shape[3] != cache.head_dim):
        raise ValueError("k_new/v_new must be [B][Hkv][n_max][D]")
    if flags is not None:
        _need(flags, "flags", U32)
        if flags.numel() != B:
            raise ValueError("flags must hold B words")
    cd = cache.desc()
    rc = lib().pa_cache_append(ctypes.byref(cd), ctypes.byref(sd), _ptr(n_new), k_new.shape[2],
                               _ptr(k_new), _ptr(v_new), _ptr(flags), _stream(stream))
    if rc != 0:
        raise PAError(rc, "pa_cache_append")


def workspace_bytes(cache, block_table, lens, num_q_heads, num_partitions=0):
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_decode_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                        num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(-1, "pa_decode_workspace_bytes")
    return n


def num_partitions(cache, block_table, lens, num_q_heads, num_partitions=0):
    """pa_decode_num_partitions: the count given, 1 for automatic on tables of at
    most 32 pages, else 0 (automatic: balanced on the device from the lengths)."""
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_decode_num_partitions(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                       num_partitions)
    if n < 0:
        raise PAError(n, "pa_decode_num_partitions")
    return n


def decode(cache, q, block_table, lens, softmax_scale, expected_tags=None, flags=None,
           num_partitions=0, out=None, workspace=None, events=None, stream=None):
    """pa_decode: q [B][Hq][D] BF16 -> out [B][Hq][D] BF16 (allocated when None)."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]")
    return _decode(cache, q, 1, block_table, lens, softmax_scale, expected_tags, flags,
                   num_partitions, out, workspace, events, stream)


def decode_noalloc(cache, q, block_table, lens, softmax_scale, expected_tags=None, flags=None,
                   num_partitions=0, out=None, stream=None):
    """pa_decode_noalloc: pa_decode with the library's static scratch in place of a
    workspace (nothing allocated by the library; `out` must be given by callers
    that cannot allocate either)."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]")
    sd = _seq(cache, block_table, lens, expected_tags)
    _need(q, "q", BF16)
    if q.shape[0] != block_table.shape[0] or q.shape[-1] != cache.head_dim:
        raise ValueError("q must be [B][Hq][D] with the table's B and the cache's D")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", BF16)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if flags is not None:
        _need(flags, "flags", U32)
        if flags.numel() != block_table.shape[0]:
            raise ValueError("flags must hold B words")
    cd = cache.desc()
    rc = lib().pa_decode_noalloc(ctypes.byref(cd), ctypes.byref(sd), q.shape[1], _ptr(q),
                                 _ptr(out), float(softmax_scale), num_partitions, _ptr(flags),
                                 _stream(stream))
    if rc != 0:
        raise PAError(rc, "pa_decode_noalloc")
    return out


def decode_step(cache, q, block_table, lens_old, n_new, k_new, v_new, lens, softmax_scale,
                expected_tags=None, flags=None, num_partitions=0, out=None, workspace=None,
                events=None, stream=None):
    """pa_decode_step: append k_new/v_new [B][Hkv][n_max][D] (n_new[u] tokens at
    lens_old[u]), then decode q [B][Hq][D] (or multi-query [B][T][Hq][D]) over
    lens; the same result as append() then decode() / decode_multi()."""
    multi = q.dim() == 4
    if q.dim() not in (3, 4):
        raise ValueError("q must be [B][Hq][D] or [B][T][Hq][D]")
    q_len = q.shape[1] if multi else 1
    sd = _seq(cache, block_table, lens, expected_tags)
    for t, name in ((lens_old, "lens_old"), (n_new, "n_new")):
        _need(t, name, I32)
        if tuple(t.shape) != tuple(lens.shape):
            raise ValueError("%s must have the shape of lens" % name)
    _need(k_new, "k_new", BF16)
    _need(v_new, "v_new", BF16)
    B = block_table.shape[0]
    if (k_new.dim() != 4 or tuple(k_new.shape) != tuple(v_new.shape) or k_new.shape[0] != B
            or k_new.shape[1] != cache.num_kv_heads or k_new.shape[3] != cache.head_dim):
        raise ValueError("k_new/v_new must be [B][Hkv][n_max][D]")
    _need(q, "q", BF16)
    if q.shape[0] != B or q.shape[-1] != cache.head_dim:
        raise ValueError("q must be [B](...)[Hq][D] with the table's B and the cache's D")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", BF16)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if flags is not None:
        _need(flags, "flags", U32)
        if flags.numel() != B:
            raise ValueError("flags must hold B words")
    Hq = q.shape[-2]
    need = (multi_workspace_bytes(cache, block_table, lens, Hq, q_len, num_partitions) if multi
            else workspace_bytes(cache, block_table, lens, Hq, num_partitions))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    cd = cache.desc()
    args = (ctypes.byref(cd), ctypes.byref(sd), _ptr(lens_old), _ptr(n_new), k_new.shape[2],
            _ptr(k_new), _ptr(v_new), Hq, q_len, _ptr(q), _ptr(out), float(softmax_scale),
            num_partitions, _ptr(flags), ws_ptr, ws_bytes, _stream(stream))
    if events is None:
        rc = lib().pa_decode_step(*args)
    else:
        for e in events:
            if e is not None and not e.cuda_event:
                e.record()
        ev = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
        rc = lib().pa_decode_step_timed(*args, ev)
    if rc != 0:
        raise PAError(rc, "pa_decode_step")
    return out


def decode_scored(cache, q, block_table, lens, softmax_scale, scores, expected_tags=None,
                  flags=None, num_partitions=0, out=None, workspace=None, events=None, stream=None):
    """pa_decode_scored: pa_decode, plus each token's attention mass (summed over the
    query heads of its KV head) added to `scores` (fp32 [P][heads][S], see new_scores)."""
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][D]")
    heads = cache.num_kv_heads if cache.layout == "seq" else 1
    _need(scores, "scores", (torch.float32,))
    if tuple(scores.shape) != (cache.num_pages, heads, PAGE_SIZE):
        raise ValueError("scores must be [P][%d][%d] fp32" % (heads, PAGE_SIZE))
    return _decode(cache, q, 1, block_table, lens, softmax_scale, expected_tags, flags,
                   num_partitions, out, workspace, events, stream, scores=scores)


def scored_workspace_bytes(cache, block_table, lens, num_q_heads, num_partitions=0):
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_decode_scored_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                               num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(-1, "pa_decode_scored_workspace_bytes")
    return n


def compact(cache, block_table, lens, keep, n_keep, new_table, scores=None, flags=None,
            stream=None):
    """pa_cache_compact: write each unit's kept tokens (keep [B][Hkv][K] positions, n_keep
    shaped like lens) in order into the pages of new_table (the table's shape)."""
    sd = _seq(cache, block_table, lens)
    _need(keep, "keep", I32)
    _need(n_keep, "n_keep", I32)
    _need(new_table, "new_table", I32)
    B = block_table.shape[0]
    if keep.dim() != 3 or keep.shape[0] != B or keep.shape[1] != cache.num_kv_heads:
        raise ValueError("keep must be [B][Hkv][K]")
    if tuple(n_keep.shape) != tuple(lens.shape) or tuple(new_table.shape) != tuple(block_table.shape):
        raise ValueError("n_keep must have lens' shape and new_table the table's")
    if scores is not None:
        _need(scores, "scores", (torch.float32,))
    if flags is not None:
        _need(flags, "flags", U32)
        if flags.numel() != B:
            raise ValueError("flags must hold B words")
    cd = cache.desc()
    rc = lib().pa_cache_compact(ctypes.byref(cd), ctypes.byref(sd), _ptr(keep), keep.shape[2],
                                _ptr(n_keep), _ptr(new_table), _ptr(scores), _ptr(flags),
                                _stream(stream))
    if rc != 0:
        raise PAError(rc, "pa_cache_compact")


def decode_multi(cache, q, block_table, lens, softmax_scale, expected_tags=None, flags=None,
                 num_partitions=0, out=None, workspace=None, events=None, stream=None):
    """pa_decode_multi: q [B][T][Hq][D] BF16 (T draft tokens, the last T of each unit,
    already appended) -> out [B][T][Hq][D] BF16; draft t sees tokens 0 .. L - T + t."""
    if q.dim() != 4:
        raise ValueError("q must be [B][T][Hq][D]")
    return _decode(cache, q, q.shape[1], block_table, lens, softmax_scale, expected_tags, flags,
                   num_partitions, out, workspace, events, stream)


def prefill(cache, q, block_table, lens, softmax_scale, expected_tags=None, flags=None,
            num_partitions=0, out=None, workspace=None, events=None, stream=None):
    """pa_prefill: q [B][C][Hq][D] BF16 (a chunk of C prompt tokens, the last C of each unit,
    already appended) -> out [B][C][Hq][D] BF16; token t sees tokens 0 .. L - C + t."""
    if q.dim() != 4:
        raise ValueError("q must be [B][C][Hq][D]")
    return _decode(cache, q, q.shape[1], block_table, lens, softmax_scale, expected_tags, flags,
                   num_partitions, out, workspace, events, stream, prefill=True)


def prefill_workspace_bytes(cache, block_table, lens, num_q_heads, chunk_len, num_partitions=0):
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_prefill_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                         chunk_len, num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(-1, "pa_prefill_workspace_bytes")
    return n


def prefill_num_partitions(cache, block_table, lens, num_q_heads, chunk_len, num_partitions=0):
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_prefill_num_partitions(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                        chunk_len, num_partitions)
    if n < 0:
        raise PAError(n, "pa_prefill_num_partitions")
    return n


def multi_workspace_bytes(cache, block_table, lens, num_q_heads, q_len, num_partitions=0):
    sd = _seq(cache, block_table, lens)
    cd = cache.desc()
    n = lib().pa_decode_multi_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), num_q_heads,
                                              q_len, num_partitions)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(-1, "pa_decode_multi_workspace_bytes")
    return n


def _decode(cache, q, q_len, block_table, lens, softmax_scale, expected_tags, flags,
            num_partitions, out, workspace, events, stream, scores=None, prefill=False):
    sd = _seq(cache, block_table, lens, expected_tags)
    _need(q, "q", BF16)
    if q.shape[0] != block_table.shape[0] or q.shape[-1] != cache.head_dim:
        raise ValueError("q must be [B](...)[Hq][D] with the table's B and the cache's D")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", BF16)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    if flags is not None:
        _need(flags, "flags", U32)
        if flags.numel() != block_table.shape[0]:
            raise ValueError("flags must hold B words")
    cd = cache.desc()
    Hq = q.shape[-2]
    L = lib()
    if prefill:
        need = L.pa_prefill_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), Hq, q_len,
                                            num_partitions)
    elif scores is not None:
        need = L.pa_decode_scored_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), Hq,
                                                  num_partitions)
    elif q_len == 1:
        need = L.pa_decode_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), Hq, num_partitions)
    else:
        need = L.pa_decode_multi_workspace_bytes(ctypes.byref(cd), ctypes.byref(sd), Hq, q_len,
                                                 num_partitions)
    if need == ctypes.c_size_t(-1).value:
        raise PAError(-1, "pa_decode workspace size")
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _ptr(workspace) if need else None
    ws_bytes = workspace.numel() * workspace.element_size() if need else 0
    args = (ctypes.byref(cd), ctypes.byref(sd), Hq)
    tail = (_ptr(q), _ptr(out), float(softmax_scale), num_partitions, _ptr(flags), ws_ptr,
            ws_bytes, _stream(stream))
    if prefill:
        if events is None:
            rc = L.pa_prefill(*args, q_len, *tail)
        else:
            for e in events:
                if e is not None and not e.cuda_event:
                    e.record()
            ev = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
            rc = L.pa_prefill_timed(*args, q_len, *tail, ev)
    elif scores is not None:
        tail_s = tail[:5] + (_ptr(scores),) + tail[5:]
        if events is None:
            rc = L.pa_decode_scored(*args, *tail_s)
        else:
            for e in events:
                if e is not None and not e.cuda_event:
                    e.record()
            ev = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
            rc = L.pa_decode_scored_timed(*args, *tail_s, ev)
    elif events is None:
        if q_len == 1:
            rc = L.pa_decode(*args, *tail)
        else:
            rc = L.pa_decode_multi(*args, q_len, *tail)
    else:
        for e in events:
            if e is not None and not e.cuda_event:
                e.record()  # torch creates the underlying hipEvent on first record
        ev = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
        if q_len == 1:
            rc = L.pa_decode_timed(*args, *tail, ev)
        else:
            rc = L.pa_decode_multi_timed(*args, q_len, *tail, ev)
    if rc != 0:
        raise PAError(rc, "pa_decode_multi" if q_len > 1 else "pa_decode")
    return out


def probe_stream(buf, waves, sink, stream=None):
    """HBM read probe (pa_probe.h): read the uint8 device buffer `buf` once."""
    _need(buf, "buf", (torch.uint8,))
    _need(sink, "sink", U32)
    if sink.numel() < waves:
        raise ValueError("sink needs %d words" % waves)
    rc = lib().pa_probe_stream(_ptr(buf), buf.numel(), waves, _ptr(sink), _stream(stream))
    if rc != 0:
        raise PAError(rc, "pa_probe_stream")


def probe_gather(pool, ids, waves, block_bytes, inflight, sink, stream=None):
    """HBM read probe (pa_probe.h): wave w reads the blocks ids[w] names."""
    _need(pool, "pool", (torch.uint8,))
    _need(ids, "ids", I32)
    _need(sink, "sink", U32)
    if ids.dim() != 2 or ids.shape[0] != waves:
        raise ValueError("ids must be [waves][ids_per_wave]")
    if sink.numel() < waves:
        raise ValueError("sink needs %d words" % waves)
    rc = lib().pa_probe_gather(_ptr(pool), pool.numel(), _ptr(ids), waves, ids.shape[1],
                               block_bytes, inflight, _ptr(sink), _stream(stream))
    if rc != 0:
        raise PAError(rc, "pa_probe_gather")


def version():
    return lib().pa_version()


class DecodeStepGraph:
    """One decode step (append, then decode or multi-query decode) captured as a HIP
    graph and replayed.

    The Infire page ("How we built the most efficient inference engine for
    Cloudflare's network", section "Rust-precise CUDA kernels") keeps one graph
    per batch size so back-to-back kernels launch as one construct.  The library
    allocates nothing and issues no memsets, so its launches capture as they
    are; every buffer (cache, tables, lengths, q, out, flags, workspace) is
    fixed at capture time and read again at each replay, so the caller updates
    their contents in place between replays (new tokens, lengths, tables).
    """

    def __init__(self, cache, block_table, lens_old, n_new, k_new, v_new, q, lens,
                 softmax_scale, expected_tags=None, flags=None, num_partitions=0, warmup=1):
        self.args = (cache, block_table, lens_old, n_new, k_new, v_new, q, lens, softmax_scale,
                     expected_tags, flags, num_partitions)
        self.out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        if q.dim() == 3:
            need = workspace_bytes(cache, block_table, lens, q.shape[1], num_partitions)
        elif q.shape[1] > 8:
            need = prefill_workspace_bytes(cache, block_table, lens, q.shape[2], q.shape[1],
                                           num_partitions)
        else:
            need = multi_workspace_bytes(cache, block_table, lens, q.shape[2], q.shape[1],
                                         num_partitions)
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):       # warm up off the capture, as torch requires
            for _ in range(warmup):
                self._step()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._step()

    def _step(self):
        (cache, bt, lens_old, n_new, k_new, v_new, q, lens, scale, exp, flags, parts) = self.args
        if q.dim() == 3 or q.shape[1] <= 8:     # decode / multi-query: one call, three launches
            decode_step(cache, q, bt, lens_old, n_new, k_new, v_new, lens, scale,
                        expected_tags=exp, flags=flags, num_partitions=parts, out=self.out,
                        workspace=self.workspace)
            return
        append(cache, bt, lens_old, n_new, k_new, v_new)
        prefill(cache, q, bt, lens, scale, expected_tags=exp, flags=flags, num_partitions=parts,
                out=self.out, workspace=self.workspace)

    def replay(self):
        self.graph.replay()
        return self.out
