"""Benchmark of one paged-decode step on one MI355X.

A step is the whole hot path for one batch: the append of the step's new
token for every (sequence, KV head), then the decode (page-tag validation,
split-K attention, partition reduce), made as one pa_decode_step call: the
append shares the validation's launch, so a step is three launches
(--separate-append: pa_cache_append then pa_decode, four launches).  Inputs
are synthetic and seeded (decode_attention_paged_pa_amd.workloads) and
resident in HBM before timing.

Default workload: the 70B-shaped FP8 layer, B 64, 64 query / 8 KV heads,
D 128, 32768 tokens per sequence (4.29 GB of FP8 KV), split-K 8, tag check on.

Timing: W untimed warm-up steps; then K steps, each preceded (outside the
timed events) by a 1 GiB write that evicts L2 and the 256 MB Infinity Cache;
HIP events on the launch stream bracket each step.  The K steps are also
bracketed by device synchronisation for a wall-clock figure.  A second pass
of K steps records events between the kernels as well, for the per-kernel
split and the attention kernel's roofline (an event between two kernels
costs a few microseconds itself, so the timed steps carry none).

Prints one JSON line.  `value` is the achieved HBM GB/s of the step
(algorithmic bytes / mean step time; `step_ms` adds the median, p10 and p90);
`roofline` is the attention kernel against the 8 TB/s HBM peak;
`measured_ceiling` is what this GPU reads per second with the library's read
probes (pa_probe.h: a 4 GiB contiguous stream, and gathers of random 2 KiB
blocks), and the attention kernel's share of the gather ceiling;
`cpu_baseline` is the fp64 oracle's decode on a bounded sample of the same
workload, on this host's cores.  `graph` is the same step captured once as a
HIP graph and replayed K times (one graph launch per step instead of three
kernel launches).  --ceiling-only runs the probes alone.

--q-len T (2..8) turns the step into a multi-query step (speculative
verification): the append writes T draft tokens per unit and
pa_decode_multi attends them causally; tokens/s then counts verified tokens.
--scored makes the decode a scored decode (eviction scores updated in place).
--compact F times pa_cache_compact keeping a fraction F of every unit's
tokens (random positions) into spare pages, and reports its GB/s instead.
--prefill C times a chunked-prefill step (append of a C-token chunk, then
pa_prefill) on a Llama-3.1-8B-shaped BF16 layer: 4 sequences whose cached
prefixes are 0, 2K, 8K and 30K tokens; it reports TFLOP/s against the MFMA
bf16 peak.  --prefill-kv fp8 runs the same step over an FP8 cache (the K and V
pages widened to the bf16 / f16 MFMA operands in registers).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and decode tokens/s"
HBM_PEAK_GBS = 8000.0
FLUSH_BYTES = 1 << 30           # write before each timed step: evicts L2 and the Infinity Cache
CEILING_BYTES = 4 << 30         # the read probes' buffer
CPU_WORKERS = 16                # the host cores one GPU's share of the box gives the oracle
MFMA_BF16_PEAK_TFLOPS = 2500.0
PREFILL_PREFIXES = (0, 2048, 8192, 30720)


def prefill_flops(w):
    """Multiply-adds of the chunk's attention, x2: query t of a unit with L tokens
    sees L - C + t + 1 of them, and costs 2*D for q.k plus 2*D for p*v per token."""
    import numpy as np

    C = w.q_len
    L = w.lens.astype(np.int64).reshape(-1)
    per_unit = [int((L_u - C) * C + C * (C + 1) // 2) for L_u in L]   # sum over t of visible tokens
    heads_per_unit = w.Hq if w.layout == "seq" else w.G
    return 4 * w.D * heads_per_unit * sum(per_unit)


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def algorithmic_bytes(w, check=True, scored=False):
    """Bytes the method must move for one decode step (append + decode).

    Decode: every attended token's K and V once (L x Hkv_u x D x 2 x e), Q in and
    O out (BF16), one table entry per page read, FP8 scales per (page, head),
    and with the check on the expected and current tag per page plus the flags.
    Append: the new token's BF16 K/V in and its cached K/V out.
    """
    import numpy as np

    e = 1 if w.kv_dtype == "fp8" else 2
    T = w.q_len
    L = w.lens.astype(np.int64)
    hkv_u = w.Hkv if w.layout == "seq" else 1
    pages = (-(-L // w.S)).sum()
    kv = int(L.sum()) * hkv_u * w.D * 2 * e
    qo = 2 * w.B * T * w.Hq * w.D * 2
    table = 4 * int(pages)
    scales = 8 * int(pages) * hkv_u if e == 1 else 0
    tags = (8 * int(pages) + 4 * w.B) if check else 0
    n_units = w.B * w.Hkv
    append = n_units * T * w.D * 2 * (2 + e)
    attn = kv + w.B * T * w.Hq * w.D * 2 + table + scales
    score = 8 * int(L.sum()) * hkv_u if scored else 0     # read-modify-write of one fp32 per token
    out = dict(kv=kv, decode=kv + qo + table + scales + tags + score, append=append,
               step=kv + qo + table + scales + tags + append + score, attention_kernel=attn,
               scores=score)
    if scored:   # the score pass: K again, Q, the table, K scales, the scores read and written
        out["score_pass"] = kv // 2 + w.B * T * w.Hq * w.D * 2 + table + scales // 2 + score
    return out


def compaction_bytes(w, n_keep_units):
    """Bytes pa_cache_compact must move: every kept token's K and V read and
    written once (plus, for FP8, the source scales read and the new ones written)."""
    e = 1 if w.kv_dtype == "fp8" else 2
    kept = int(n_keep_units.sum())
    b = 2 * kept * w.D * 2 * e
    if e == 1:
        b += 2 * 4 * kept + 2 * 4 * -(-kept // w.S)
    return b


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("pa_decode.hip", "pa_device.h", "pa_internal.h", "pa_block.h"):
        with open(os.path.join(ROOT, "decode_attention_paged_pa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name, per_launch_units):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_attention_%s.json" % name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- CPU baseline
def _oracle_worker(w, seqs, barrier, queue):
    import numpy as np  # noqa: F401

    from oracle import oracle_decode, oracle_decode_multi
    from tests.oracle_fill import oracle_fill

    run = oracle_decode if w.q_len == 1 else oracle_decode_multi
    cache, _ = oracle_fill(w, seqs=seqs)           # untimed: building the cache
    barrier.wait()
    t0 = time.perf_counter()
    for b in seqs:
        run(cache, w.q[b:b + 1], w.block_table[b:b + 1], w.lens[b:b + 1], w.sigma)
    queue.put(time.perf_counter() - t0)


def cpu_baseline(w, n_seqs):
    import multiprocessing as mp

    ctx = mp.get_context("spawn")
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(CPU_WORKERS, affinity, n_seqs))
    step = max(1, w.B // n_seqs)
    sample = list(range(0, w.B, step))[:n_seqs]
    shares = [sample[i::cores] for i in range(cores)]
    barrier = ctx.Barrier(cores + 1)
    queue = ctx.Queue()
    env_threads = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                    "MKL_NUM_THREADS")}
    for k in env_threads:
        os.environ[k] = "1"
    procs = [ctx.Process(target=_oracle_worker, args=(w, s, barrier, queue)) for s in shares]
    for p in procs:
        p.start()
    for k, v in env_threads.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    barrier.wait()
    t0 = time.perf_counter()
    times = [queue.get(timeout=600) for _ in procs]
    wall = time.perf_counter() - t0
    for p in procs:
        p.join()
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except Exception:
        pass
    fn = "oracle_decode" if w.q_len == 1 else "oracle_decode_multi (%d drafts)" % w.q_len
    per = sorted(set(len(x) for x in shares))
    return dict(value=len(sample) * w.q_len / wall, unit="tokens/s", cores=cores, kind="oracle",
                sample="%s (gather, FP8 dequant, fp64 attention) of %d of the %d "
                       "sequences (all %d query heads each) of the same workload, %s per worker "
                       "process (one thread each), cache build untimed; %.1f s of CPU decode "
                       "work; %s" % (fn, len(sample), w.B, w.Hq,
                                     " or ".join(str(x) for x in per), sum(times), cpu_model),
                seconds_wall=wall, host_affinity_cores=affinity,
                cores_note="%d worker processes: one GPU's share of the box's host cores "
                           "(%d visible to the process)" % (cores, affinity))


# ---------------------------------------------------------------- read ceiling
def _timed(fn, stream, flush, reps):
    """Median ms of `reps` calls of fn, each after the flush write, by HIP events."""
    import numpy as np
    import torch

    ts = []
    for _ in range(reps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def measure_ceilings(dev, flush, reps=5, log_fn=None):
    """What this GPU reads per second (pa_probe.h), best over the probes' launch shapes:
    a contiguous read of CEILING_BYTES; a gather of every 2 KiB block of that
    buffer in random order (2048 waves, one run of blocks each); and the
    decode's own SEQ pattern, pages of 8 head blocks (16 KiB) in random order
    whose 8 blocks are read by 8 waves on one XCD."""
    import numpy as np
    import torch

    from decode_attention_paged_pa_amd import pa

    stream = torch.cuda.current_stream()
    buf = torch.empty(CEILING_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)
    out = {}
    best = (0.0, None)
    for waves in (2048, 8192, 16384):
        ms = _timed(lambda: pa.probe_stream(buf, waves, sink, stream), stream, flush, reps)
        gbs = CEILING_BYTES / (ms * 1e-3) / 1e9
        best = max(best, (gbs, "%d waves" % waves))
    out["stream_read"] = {"GB/s": round(best[0], 1), "bytes": CEILING_BYTES, "config": best[1]}
    rng = np.random.default_rng(99)
    nblk = CEILING_BYTES // 2048
    waves = 2048
    # random 2 KiB blocks, every block once
    ids = torch.from_numpy(rng.permutation(nblk).astype(np.int32).reshape(waves, -1)).to(dev)
    # SEQ pages: 8 consecutive 2 KiB blocks (one per KV head) in random page order; the
    # 8 waves of a page run are the 4 waves of workgroups x and x + 8 (one XCD)
    npg = nblk // 8
    runs = waves // 8
    order = rng.permutation(npg).astype(np.int64).reshape(runs, -1)
    page_ids = np.empty((waves, order.shape[1]), np.int32)
    for r in range(runs):
        for h in range(8):
            wg = (r // 8) * 16 + (h // 4) * 8 + r % 8
            page_ids[wg * 4 + h % 4] = (order[r] * 8 + h).astype(np.int32)
    page_ids = torch.from_numpy(page_ids).to(dev)
    for name, tab in (("gather_2KiB", ids), ("gather_2KiB_seq_pages", page_ids)):
        best = (0.0, None)
        for inflight in (1, 2, 4):
            ms = _timed(lambda: pa.probe_gather(buf, tab, waves, 2048, inflight, sink, stream),
                        stream, flush, reps)
            gbs = (nblk * 2048 + nblk * 4) / (ms * 1e-3) / 1e9
            if log_fn:
                log_fn("%s inflight %d: %.3f ms, %.0f GB/s" % (name, inflight, ms, gbs))
            best = max(best, (gbs, "%d waves, %d blocks in flight per wave" % (waves, inflight)))
        out[name] = {"GB/s": round(best[0], 1), "bytes": nblk * 2048 + nblk * 4, "config": best[1]}
    del buf, ids, page_ids
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------- compaction
def bench_compaction(args):
    """pa_cache_compact on a workload with enough spare pages: every unit keeps a
    random fraction of its tokens (increasing positions), written to fresh pages."""
    import numpy as np
    import torch

    from decode_attention_paged_pa_amd import pa
    from decode_attention_paged_pa_amd.device_inputs import build_device_workload
    from decode_attention_paged_pa_amd.workloads import make_workload

    frac = args.compact
    probe = make_workload(args.config, stale_frac=0.0)
    used = probe.n_pages_used()
    w = make_workload(args.config, stale_frac=0.0,
                      spare_pages=int(used * frac) + probe.B * probe.Hkv + 64)
    log("compaction to %.4f of the tokens: workload %d %s, P=%d" % (frac, w.cfg_id, w.name, w.P))
    dw = build_device_workload(w, threads=args.threads, log=log)
    dw.step_append()
    rng = np.random.default_rng(7)
    lens_u = w.lens.reshape(-1) if w.layout == "head" else np.repeat(w.lens, w.Hkv)
    if w.layout == "seq":
        n_keep = np.maximum(1, (w.lens * frac).astype(np.int32))
        n_units = np.repeat(n_keep, w.Hkv)
    else:
        n_keep = np.maximum(1, (w.lens * frac).astype(np.int32))
        n_units = n_keep.reshape(-1)
    K = int(n_units.max())
    keep = np.zeros((w.B * w.Hkv, K), np.int32)
    for u in range(w.B * w.Hkv):
        n = int(n_units[u])
        keep[u, :n] = np.sort(rng.choice(int(lens_u[u]), n, replace=False))
    keep = keep.reshape(w.B, w.Hkv, K)
    used_pages = set(w.block_table[w.block_table != 0x7FFFFFFF].tolist())
    free = np.array([p for p in range(w.P) if p not in used_pages], np.int32)
    nt = np.full(w.block_table.shape, 0x7FFFFFFF, np.int32)
    k = 0
    rows = [(b,) for b in range(w.B)] if w.layout == "seq" else [
        (b, h) for b in range(w.B) for h in range(w.Hkv)]
    for row in rows:
        need = -(-int(n_keep[row]) // w.S)
        nt[row][:need] = free[k:k + need]
        k += need
    keep_d = torch.from_numpy(keep).cuda()
    n_keep_d = torch.from_numpy(n_keep.astype(np.int32)).cuda()
    nt_d = torch.from_numpy(nt).cuda()
    scores = dw.cache.new_scores()
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for _ in range(args.warmup):
        pa.compact(dw.cache, dw.block_table, dw.lens, keep_d, n_keep_d, nt_d, scores=scores)
    torch.cuda.synchronize()
    ts = []
    for _ in range(args.steps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pa.compact(dw.cache, dw.block_table, dw.lens, keep_d, n_keep_d, nt_d, scores=scores)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.mean(ts))
    by = compaction_bytes(w, n_units) + 8 * int(n_units.sum())   # + the scores moved
    gbs = by / (ms * 1e-3) / 1e9
    log("compaction: %.3f ms, %d tokens kept of %d, %.0f GB/s (%.1f%% of 8 TB/s)" % (
        ms, int(n_units.sum()), int(lens_u.sum()), gbs, gbs / 80))
    print(json.dumps({
        "metric": "KV compaction after eviction: achieved HBM GB/s", "value": round(gbs, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.kv_dtype, "data": "synthetic",
        "config": {"workload": "%s, keep %.4f of every unit's tokens (random positions), "
                               "scores moved" % (w.name, frac), "global_batch": w.B},
        "algorithmic_bytes": by,
        "roofline": {"bound": "hbm", "kernel": "compact_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "cpu_baseline": None}), flush=True)


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="workload: 2 llama8b-bf16, 3 llama8b-fp8-tags, 4 headwise-bf16, "
                         "5 70b-fp8-32k (B 64, 64/8 heads, D 128, 32K tokens, FP8)")
    ap.add_argument("--partitions", type=int, default=-1,
                    help="split-K count (-1: 8 for the 70b-fp8-32k decode, else the library's "
                         "choice)")
    ap.add_argument("--no-check", action="store_true", help="no-op tracker: skip the tag check")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="keep this many KV heads (and their query heads) of the workload: one "
                         "GPU's share of the layer when its KV heads are sharded over GPUs")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=32, help="sequences in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--threads", type=int, default=16)
    ap.add_argument("--q-len", type=int, default=1,
                    help="draft tokens per sequence (multi-query step), 1..8")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--separate-append", action="store_true",
                    help="append and decode as two calls (four launches) instead of pa_decode_step")
    ap.add_argument("--scored", action="store_true", help="scored decode (eviction scores)")
    ap.add_argument("--compact", type=float, default=0.0,
                    help="time compaction to this fraction of the tokens instead")
    ap.add_argument("--prefill", type=int, default=0,
                    help="time a chunked-prefill step with this chunk length instead")
    ap.add_argument("--prefill-kv", choices=("bf16", "fp8"), default="bf16",
                    help="cache format of the --prefill step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter scale)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="only run the HBM read probes (pa_probe.h) and print their rates")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the HBM read probes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decode_attention_paged_pa_amd import pa
    from decode_attention_paged_pa_amd.device_inputs import build_device_workload
    from decode_attention_paged_pa_amd.workloads import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "launches": 5}))
        return
    if args.ceiling_only:
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        c = measure_ceilings(dev, flush, log_fn=log)
        print(json.dumps({"metric": "HBM read ceiling (pa_probe.h)", "measured_ceiling": c,
                          "peak": HBM_PEAK_GBS}), flush=True)
        return
    if args.compact > 0:
        return bench_compaction(args)
    if args.prefill > 0:
        C = args.prefill
        prefill_name = "llama8b-prefill" if args.prefill_kv == "bf16" else "llama8b-fp8-prefill"
        w = make_workload(2 if args.prefill_kv == "bf16" else 3, batch=len(PREFILL_PREFIXES),
                          stale_frac=0.0, q_len=C, lens=np.array(PREFILL_PREFIXES) + C,
                          table_width=2048)
    else:
        heads = None
        if args.kv_heads > 0:
            full = make_workload(args.config, stale_frac=0.0, batch=1)
            if full.Hkv % args.kv_heads:
                sys.exit("--kv-heads must divide the workload's %d KV heads" % full.Hkv)
            heads = (full.G * args.kv_heads, args.kv_heads)
        w = make_workload(args.config, stale_frac=0.0, q_len=args.q_len, heads=heads)
    # split-K 8 is the decode workload's own setting; multi-query steps take the
    # library's choice (whole grid resident: 4 on the 70B-shaped workload)
    parts = args.partitions if args.partitions >= 0 else (
        8 if args.config == 5 and args.q_len == 1 and args.prefill == 0 else 0)
    check = not args.no_check
    T = w.q_len
    log("workload %d %s: B=%d Hq=%d Hkv=%d D=%d kv=%s layout=%s tokens=%d q_len=%d" % (
        w.cfg_id, w.name, w.B, w.Hq, w.Hkv, w.D, w.kv_dtype, w.layout, int(w.lens.sum()), T))
    t0 = time.time()
    dw = build_device_workload(w, device=dev, threads=args.threads, log=log)
    dw.step_append()
    torch.cuda.synchronize()
    log("cache filled in %.1f s" % (time.time() - t0))
    n_parts = pa.num_partitions(dw.cache, dw.block_table, dw.lens, w.Hq, parts)
    if args.scored:
        ws_bytes = pa.scored_workspace_bytes(dw.cache, dw.block_table, dw.lens, w.Hq, parts)
        scores = dw.cache.new_scores()
    elif args.prefill > 0:
        ws_bytes = pa.prefill_workspace_bytes(dw.cache, dw.block_table, dw.lens, w.Hq, T, parts)
        n_parts = pa.prefill_num_partitions(dw.cache, dw.block_table, dw.lens, w.Hq, T, parts)
    else:
        ws_bytes = pa.multi_workspace_bytes(dw.cache, dw.block_table, dw.lens, w.Hq, T, parts)
    workspace = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty(tuple(dw.q.shape), dtype=torch.bfloat16, device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # a decode step is pa_decode_step (its append shares the validation's launch),
    # or, with --separate-append, the scored decode and prefill, two calls
    fused = not args.separate_append and not args.scored and args.prefill == 0

    def step(evs=None):
        if evs is not None:
            evs[0].record(stream)
        if fused:
            dw.decode_step(check=check, num_partitions=parts, out=out, workspace=workspace,
                           events=None if evs is None else evs[1:])
            return
        dw.step_append()
        if args.scored:
            pa.decode_scored(dw.cache, dw.q, dw.block_table, dw.lens, w.sigma, scores,
                             expected_tags=dw.expected_tags if check else None,
                             flags=dw.flags if check else None, num_partitions=parts, out=out,
                             workspace=workspace, events=None if evs is None else evs[1:])
        else:
            dw.decode(check=check, num_partitions=parts, out=out, workspace=workspace,
                      events=None if evs is None else evs[1:])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # Timed steps carry two events each (start, end): an event recorded
    # between kernels costs a few microseconds of its own on this stack, so
    # the per-kernel split comes from a second pass of K steps with events
    # between the launches (the same work, same flushes).
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    for e in sev + evs:
        for x in e:
            x.record(stream)   # create the underlying events before timing
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for k in range(K):
        if not args.no_flush:
            flush.zero_()
        sev[k][0].record(stream)
        step()
        sev[k][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    for k in range(K):
        if not args.no_flush:
            flush.zero_()
        step(evs[k])
    torch.cuda.synchronize()
    t_step = np.array([e[0].elapsed_time(e[1]) for e in sev])          # ms
    t_split = np.array([e[0].elapsed_time(e[4]) for e in evs])
    t_append = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_val = np.array([e[1].elapsed_time(e[2]) for e in evs])
    t_attn = np.array([e[2].elapsed_time(e[3]) for e in evs])
    t_red = np.array([e[3].elapsed_time(e[4]) for e in evs])
    ms = float(t_step.mean())
    by = algorithmic_bytes(w, check, args.scored)
    gbs = by["step"] / (ms * 1e-3) / 1e9
    attn_gbs = by["attention_kernel"] / (t_attn.mean() * 1e-3) / 1e9
    tok_s = w.B * T / (ms * 1e-3)
    log("step %.3f ms (p10 %.3f p90 %.3f; %.3f ms with events between the kernels); append "
        "%.1f us, %s %.1f us, attention %.1f us, "
        "reduce%s %.1f us; %.0f GB/s step, attention %.0f GB/s (%.1f%% of 8 TB/s)" % (
            ms, np.percentile(t_step, 10), np.percentile(t_step, 90), t_split.mean(),
            t_append.mean() * 1e3,
            "append+validate (one launch)" if fused else "validate",
            t_val.mean() * 1e3, t_attn.mean() * 1e3, " + score" if args.scored else "",
            t_red.mean() * 1e3, gbs, attn_gbs,
            100 * attn_gbs / HBM_PEAK_GBS))
    if args.scored:
        log("score pass (with the reduce): %.0f GB/s of its own bytes" % (
            by["score_pass"] / (t_red.mean() * 1e-3) / 1e9))

    graph = None
    if not args.no_graph and not args.scored and args.prefill == 0:
        g = pa.DecodeStepGraph(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step,
                               dw.v_step, dw.q, dw.lens, w.sigma,
                               expected_tags=dw.expected_tags if check else None,
                               flags=dw.flags if check else None, num_partitions=parts)
        gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
        for e in gev:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        for k in range(K):
            if not args.no_flush:
                flush.zero_()
            gev[k][0].record(stream)
            g.replay()
            gev[k][1].record(stream)
        torch.cuda.synchronize()
        g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gev]))
        graph = {"ms_per_step": round(g_ms, 4),
                 "value": round(by["step"] / (g_ms * 1e-3) / 1e9, 1),
                 "tokens_per_s": round(w.B * T / (g_ms * 1e-3), 1)}
        log("graph replay: step %.3f ms (%.0f GB/s)" % (g_ms, graph["value"]))
        del g

    prof_name = w.name if T == 1 else "%s-t%d" % (w.name, T)
    if args.kv_heads > 0:
        prof_name += "-kv%d" % args.kv_heads
    traffic = traffic_from_profile(prof_name, None)
    if args.prefill > 0:
        fl = prefill_flops(w)
        tflops = fl / (t_attn.mean() * 1e-3) / 1e12
        log("prefill: %.3g GFLOP per step; attention kernel %.1f us = %.0f TFLOP/s (%.1f%% of "
            "the %d TFLOP/s bf16 MFMA peak)" % (fl / 1e9, t_attn.mean() * 1e3, tflops,
                                                 100 * tflops / MFMA_BF16_PEAK_TFLOPS,
                                                 MFMA_BF16_PEAK_TFLOPS))
    if args.prefill > 0:
        step_tflops = fl / (ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": "chunked prefill attention over the paged cache: achieved TFLOP/s",
            "value": round(step_tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "%s: B=4, Hq=32, Hkv=8, D=128, page 16, %s KV, "
                                   "SEQ layout, cached prefixes %s, chunk %d, %d partitions, tag "
                                   "check %s" % (prefill_name, args.prefill_kv.upper(),
                                                 list(PREFILL_PREFIXES), T, n_parts,
                                                 "on" if check else "off"),
                       "global_batch": w.B, "chunk_tokens": T},
            "flops_per_step": fl,
            "kernels_us": {"append": round(t_append.mean() * 1e3, 2),
                           "validate": round(t_val.mean() * 1e3, 2),
                           "attention": round(t_attn.mean() * 1e3, 2),
                           "reduce": round(t_red.mean() * 1e3, 2)},
            "roofline": {"bound": "mfma", "kernel": "attention_kernel", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": traffic_from_profile("%s-%d" % (prefill_name, T), None)},
            "cpu_baseline": None}), flush=True)
        return
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8",
        "data": "synthetic",
        "config": {
            "workload": "%s: B=%d, Hq=%d, Hkv=%d, D=%d, page 16, L=%s, %s KV, %s layout, "
                        "split-K %s, tag check %s%s" % (
                            w.name, w.B, w.Hq, w.Hkv, w.D,
                            "32768" if args.config == 5 else "drawn",
                            "FP8 e4m3" if w.kv_dtype == "fp8" else "BF16", w.layout.upper(),
                            n_parts if n_parts > 0 else "balanced on the device",
                            "on" if check else "off",
                            ("" if T == 1 else ", %d draft tokens per sequence (causal)" % T)
                            + (", eviction scores updated" if args.scored else "")
                            + (", one GPU's share of the KV heads" if args.kv_heads > 0 else "")),
            "q_len": T,
            "global_batch": w.B,
            "tokens_attended": int(w.lens.sum()),
            "parallelism": "1 GPU",
        },
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "step_ms": {"mean": round(ms, 4), "median": round(float(np.median(t_step)), 4),
                    "p10": round(float(np.percentile(t_step, 10)), 4),
                    "p90": round(float(np.percentile(t_step, 90)), 4)},
        "tokens_per_s": round(tok_s, 1),
        "wall_ms_per_step_incl_flush": round(wall / K * 1e3, 4),
        "ms_per_step_with_kernel_events": round(float(t_split.mean()), 4),
        "kernels_us": ({"append+validate": round(t_val.mean() * 1e3, 2)} if fused else
                       {"append": round(t_append.mean() * 1e3, 2),
                        "validate": round(t_val.mean() * 1e3, 2)}) | {
                       "attention": round(t_attn.mean() * 1e3, 2),
                       ("reduce+score" if args.scored else "reduce"): round(t_red.mean() * 1e3, 2)},
        "step_calls": "pa_decode_step (3 launches)" if fused else "pa_cache_append + decode",
        "algorithmic_bytes": by,
        "graph": graph,
        "roofline": {
            "bound": "hbm",
            "kernel": "attention_kernel",
            "achieved": round(attn_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if not args.no_ceiling and args.prefill == 0:
        c = measure_ceilings(dev, flush, log_fn=log)
        c["attention_pct_of_gather_ceiling"] = round(
            100 * attn_gbs / max(c["gather_2KiB"]["GB/s"], c["gather_2KiB_seq_pages"]["GB/s"]), 2)
        c["attention_pct_of_stream_ceiling"] = round(100 * attn_gbs / c["stream_read"]["GB/s"], 2)
        result["measured_ceiling"] = c
        log("read ceiling: stream %.0f GB/s, 2 KiB gather %.0f GB/s, SEQ-page gather %.0f GB/s; "
            "attention at %.1f%% of the best gather" % (
                c["stream_read"]["GB/s"], c["gather_2KiB"]["GB/s"],
                c["gather_2KiB_seq_pages"]["GB/s"], c["attention_pct_of_gather_ceiling"]))
    del flush, workspace
    if not args.no_cpu_baseline:
        log("timing the oracle on %d sequences ..." % args.cpu_seqs)
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seqs)
        log("oracle: %.3f tokens/s on %d cores" % (result["cpu_baseline"]["value"],
                                                  result["cpu_baseline"]["cores"]))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
