"""The committed rocprofv3 traffic summaries agree with themselves and with the
byte counts bench.py prices its roofline on (no GPU needed).

Each `profiles/traffic_*.json` holds the FETCH_SIZE / WRITE_SIZE counter means
of one kernel, the copy-calibration factors, and the HBM bytes derived from
them.  These tests redo that arithmetic, recompute the algorithmic bytes from
the named workload, and check that the summary was taken on the kernel source
in the tree (bench.py reports the traffic only then).
"""
import glob
import importlib.util
import json
import os

import numpy as np
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_for_tests", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


BENCH = _bench()


def _algorithmic(name):
    """Algorithmic bytes per launch of the kernel a summary covers, from its workload name."""
    kind, wl = name.split("_", 2)[1:]
    if wl.startswith("llama8b-fp8-prefill-"):
        C = int(wl.rsplit("-", 1)[1])
        w = make_workload(3, batch=len(BENCH.PREFILL_PREFIXES), stale_frac=0.0, q_len=C,
                          lens=np.array(BENCH.PREFILL_PREFIXES) + C, table_width=2048)
        return BENCH.algorithmic_bytes(w)["attention_kernel"]
    if wl.startswith("llama8b-prefill-"):
        C = int(wl.rsplit("-", 1)[1])
        w = make_workload(2, batch=len(BENCH.PREFILL_PREFIXES), stale_frac=0.0, q_len=C,
                          lens=np.array(BENCH.PREFILL_PREFIXES) + C, table_width=2048)
        return BENCH.algorithmic_bytes(w)["attention_kernel"]
    assert wl.startswith("70b-fp8-32k"), wl
    rest = wl[len("70b-fp8-32k"):]
    if kind == "mass":
        assert rest == "-scored", wl
        w = make_workload(5, stale_frac=0.0)
        return BENCH.algorithmic_bytes(w, scored=True)["score_pass"]
    T = int(rest[2:]) if rest.startswith("-t") else 1
    assert rest in ("", "-t%d" % T), wl
    w = make_workload(5, stale_frac=0.0, q_len=T)
    return BENCH.algorithmic_bytes(w)["attention_kernel"]


def test_there_are_traffic_summaries():
    names = [os.path.basename(f) for f in FILES]
    assert "traffic_attention_70b-fp8-32k.json" in names
    assert "traffic_attention_llama8b-prefill-2048.json" in names


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(f)[:-5] for f in FILES])
def test_traffic_summary_arithmetic(path):
    d = json.load(open(path))
    for k in ("kernel", "workload", "kernel_source_sha", "commands", "fetch_size_kib_per_launch",
              "write_size_kib_per_launch", "fetch_scale", "write_scale", "hbm_read_bytes_per_launch",
              "hbm_write_bytes_per_launch", "hbm_bytes_per_launch", "algorithmic_bytes_per_launch"):
        assert k in d, k
    # the commands name a FETCH_SIZE pass, a WRITE_SIZE pass and the copy calibration
    cmds = " ".join(d["commands"])
    assert "--pmc FETCH_SIZE" in cmds and "--pmc WRITE_SIZE" in cmds and "--copy-calibration" in cmds
    # counters -> bytes: KiB x 1024 x the factor a plain 1 GiB copy needs (rounded inputs)
    rd = d["fetch_size_kib_per_launch"] * 1024 * d["fetch_scale"]
    wr = d["write_size_kib_per_launch"] * 1024 * d["write_scale"]
    assert abs(rd - d["hbm_read_bytes_per_launch"]) <= 1e-4 * rd + 1024
    assert abs(wr - d["hbm_write_bytes_per_launch"]) <= 1e-4 * wr + 1024
    # (each of the three is truncated to whole bytes on its own)
    assert abs(d["hbm_bytes_per_launch"] - d["hbm_read_bytes_per_launch"]
               - d["hbm_write_bytes_per_launch"]) <= 1
    if "copy_1GiB_fetch_size_kib" in d:
        assert d["fetch_scale"] == pytest.approx((1 << 20) / d["copy_1GiB_fetch_size_kib"], rel=1e-4)
        assert d["write_scale"] == pytest.approx((1 << 20) / d["copy_1GiB_write_size_kib"], rel=1e-4)
    # the algorithmic bytes are the ones bench.py prices the roofline on
    assert d["algorithmic_bytes_per_launch"] == _algorithmic(os.path.basename(path)[:-5])


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(f)[:-5] for f in FILES])
def test_traffic_summary_matches_kernel_source(path):
    d = json.load(open(path))
    sha = BENCH.kernel_source_sha()
    if d["kernel_source_sha"] != sha:
        pytest.skip("taken on kernel source %s, the tree has %s: bench.py reports traffic null "
                    "until the counters are taken again" % (d["kernel_source_sha"], sha))
    name = os.path.basename(path)[len("traffic_attention_"):-5]
    if os.path.basename(path).startswith("traffic_attention_"):
        assert BENCH.traffic_from_profile(name, None) == d["hbm_bytes_per_launch"]
