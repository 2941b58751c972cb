"""bench.py's command line and the counts it prices its metrics on (no GPU).

The chunked-prefill metric is TFLOP/s of causal attention: 4 D flops (q.k and
p*v, a multiply-add each) per visible (query, key) pair and query head.  Here
the pairs are counted from an explicit causal mask, not from the sum bench.py
uses.
"""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_cli_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a configuration it does not measure


@pytest.mark.parametrize("cfg", [2, 3])          # the BF16 and FP8 Llama-8B-shaped layers
@pytest.mark.parametrize("C", [16, 64, 100])
def test_prefill_flops_count_every_visible_pair(cfg, C):
    bench = _bench()
    w = make_workload(cfg, batch=4, stale_frac=0.0, q_len=C, lens=np.array([0, 40, 100, 333]) + C,
                      table_width=64)
    pairs = 0
    for L in w.lens.reshape(-1):
        t = np.arange(C)[:, None]             # chunk token t sits at position L - C + t
        j = np.arange(int(L))[None, :]        # key positions
        pairs += int(np.count_nonzero(j <= int(L) - C + t))
    assert bench.prefill_flops(w) == 4 * w.D * w.Hq * pairs


def test_prefill_workloads_share_their_flops():
    """The --prefill-kv fp8 step attends the same pairs as the BF16 one."""
    bench = _bench()
    C = 512
    lens = np.array(bench.PREFILL_PREFIXES) + C
    wb = make_workload(2, batch=len(lens), stale_frac=0.0, q_len=C, lens=lens, table_width=2048)
    wf = make_workload(3, batch=len(lens), stale_frac=0.0, q_len=C, lens=lens, table_width=2048)
    assert wb.kv_dtype == "bf16" and wf.kv_dtype == "fp8"
    assert bench.prefill_flops(wb) == bench.prefill_flops(wf)


def test_headline_attention_bytes_from_the_shape():
    """The decode metric's bytes per attention launch on the 70B-shaped FP8 layer,
    from its shape: K and V once (one byte per element), Q in BF16, the table
    entries the step reads, and the K and V scales of every (page, KV head)."""
    bench = _bench()
    w = make_workload(5, stale_frac=0.0)
    B, Hq, Hkv, D, L, S = 64, 64, 8, 128, 32768, 16
    pages = L // S
    kv = B * L * Hkv * 2 * D * 1
    q = B * Hq * D * 2
    table = B * pages * 4
    scales = B * pages * Hkv * 2 * 4
    assert bench.algorithmic_bytes(w)["attention_kernel"] == kv + q + table + scales == 4_304_928_768
