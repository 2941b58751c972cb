"""FP8 caches at magnitudes far from N(0, 1), on the GPU against the oracle.

The FP8 cache format ("Cloudflare quantizes Kimi and GLM caches for 41% faster
inference", KV cache quantization paragraph) takes any BF16 K/V: a page's
scale is fl32(amax / 448), so its codes look the same at every magnitude and
the scales carry the range.  The kernels must then keep their f16 P.V
operands inside f16's range and precision at any scale, for pages of one
magnitude and for pages whose magnitudes differ by many decades.

Pool bytes and scales are compared bit for bit.  Outputs are compared per KV
head against bars in the units of that head's values (m = max |V| over the
unit's tokens): the kernel's P.V operand carries an f16 relative error of at
most 2^-11 per weight, and the weights sum to 1, so the P rounding moves an
output by at most 2^-11 m; the BF16 output rounding adds at most 2^-9 |o| <=
2^-9 m.  The bars are max |err| <= 2^-8 m and mean |err| <= 2^-12 m +
2^-9 mean |o|: for N(0, 1) values averaged over many tokens, m is about 4.5
and |o| well below 1, so these are about 1.8e-2 and 1.1e-3, the usual 1e-2 /
1e-3 bars in that head's units; the second mean term is the output's own
rounding, which is all the error there is where a unit holds one token (the
output is then one V row).  Where K and V are scaled by one constant f, the
usual bars times f apply as well.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from oracle import bf16_to_f64
from tests.oracle_fill import oracle_sequences_parallel
from tests.test_gpu_parity import compare_pools, flags_of, log, out_f64

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 2.0 ** -8, 2.0 ** -12


def unit_vmax(w, b):
    """max |V| per KV head of sequence b, from the generator's draws."""
    k_hist, v_hist, k_new, v_new, n_hist = w.seq_kv(b)
    m = np.zeros(w.Hkv)
    for h in range(w.Hkv):
        n = int(n_hist[h])
        v = np.concatenate([bf16_to_f64(v_hist[h, :n]).ravel(), bf16_to_f64(v_new[h]).ravel()])
        m[h] = np.max(np.abs(v)) if v.size else 0.0
    return m


def check_rows(w, out, ora, seqs, flags, const=None, what=""):
    """Per-head relative bars (module notes); const: the usual bars times const."""
    got = out_f64(out)
    worst = 0.0
    for b in seqs:
        if flags is not None and flags[b] != 0:
            assert np.all(out[b].view(torch.int16).cpu().numpy() == 0)
            continue
        vmax = unit_vmax(w, b)
        g, r = got[b], ora[b]["out"]            # [Hq][D] or [T][Hq][D]
        assert np.all(np.isfinite(g)), b
        err = np.abs(g - r).reshape(-1, w.Hq, w.D)
        for h in range(w.Hkv):
            e = err[:, h * w.G:(h + 1) * w.G, :]
            m = vmax[h]
            assert e.max() <= MAX_REL * m, (what, b, h, e.max(), m)
            o_mean = np.abs(r).reshape(-1, w.Hq, w.D)[:, h * w.G:(h + 1) * w.G, :].mean()
            assert e.mean() <= MEAN_REL * m + 2.0 ** -9 * o_mean, (what, b, h, e.mean(), m)
            worst = max(worst, e.max() / m if m else 0.0)
            if const is not None:
                assert e.max() <= 1e-2 * const and e.mean() <= 1e-3 * const, (what, b, h)
    log("%s worst max-abs / max|V| = %.3g" % (what, worst))


def run_range_case(w, partitions=(0,), const=None, pools=True):
    log("fp8 range: %s kv_mag=%s B=%d T=%d lens=%s sigma=%g" % (
        w.layout, w.kv_mag, w.B, w.q_len, w.lens.ravel()[:6].tolist(), w.sigma))
    dw = build_device_workload(w)
    dw.step_append()
    seqs = list(range(w.B))
    ora = oracle_sequences_parallel(w, seqs)
    if pools:
        compare_pools(dw, ora, seqs)
    for p in partitions:
        out = dw.decode(check=True, num_partitions=p)
        torch.cuda.synchronize()
        fl = flags_of(dw)
        assert np.all(fl == 0)
        check_rows(w, out, ora, seqs, fl, const, "partitions=%d" % p)


LENS = [300, 1500, 4100, 9000]


@pytest.mark.parametrize("which,f", [("v", 1e-6), ("v", 1e-3), ("v", 1e5), ("k", 1e-3),
                                     ("k", 1e5), ("kv", 1e-3), ("kv", 1e5)])
def test_constant_magnitudes(which, f):
    """K and/or V times one constant; when K is scaled the softmax scale is
    divided by the same factor, so the weights are those of the N(0, 1) draws."""
    mag = {c: f for c in which}
    sigma = (1.0 / np.sqrt(128)) / (f if "k" in which else 1.0)
    w = make_workload(3, batch=4, lens=LENS, stale_frac=0.0, kv_mag=mag, sigma=sigma)
    run_range_case(w, partitions=(0, 1, 3), const=f if "v" in which else 1.0)


def test_pages_of_mixed_magnitudes():
    """Every page of every unit at its own magnitude, 10^-4 .. 10^4, K and V
    drawn apart: the largest-scale pages dominate the scores (near one-hot
    weights) and the V operands span eight decades within a segment."""
    w = make_workload(3, batch=4, lens=LENS, stale_frac=0.0,
                      kv_mag={"k": ("pages", -1, 1), "v": ("pages", -4, 4)})
    run_range_case(w, partitions=(0, 1, 3))


def test_magnitude_growing_along_the_sequence():
    """V grows by 8 decades along each unit, so a wave's reference scale grows at
    every 256-page segment of a long run (one partition: runs of 1024 pages)."""
    w = make_workload(3, batch=3, lens=[16384, 9000, 4500], stale_frac=0.0,
                      kv_mag={"v": ("ramp", -4, 4)})
    run_range_case(w, partitions=(0, 1, 2))


def test_growth_after_a_parked_partition():
    """A wave that streams two partitions parks the first one's state until the
    end; with V growing along the unit its reference scale grows after the
    park.  64 KV heads (G = 1) x 32 sequences makes 2048 units, so two
    partitions of 257 pages go to one wave (runs over 3 segments)."""
    L = 16 * 513
    w = make_workload(3, batch=32, lens=[L] * 32, heads=(64, 64), head_dim=64,
                      table_width=514, stale_frac=0.0, kv_mag={"v": ("ramp", -3, 4)})
    run_range_case(w, partitions=(2,), pools=False)


@pytest.mark.parametrize("T,heads", [(4, (64, 8)), (8, (64, 8)), (2, (32, 8))])
def test_multi_query_magnitudes(T, heads):
    """The multi-tile kernels (2 and 4 column tiles): V at 1e5, and V growing
    along the unit."""
    for mag in ({"v": 1e5}, {"v": ("ramp", -3, 4)}):
        w = make_workload(5, batch=3, lens=[40, 3000, 9000], q_len=T, heads=heads,
                          table_width=600, stale_frac=0.0, kv_mag=mag)
        run_range_case(w, partitions=(0, 3))


def test_prefill_chunk_magnitudes():
    """A 96-token prefill chunk (384 columns: the page-sharing kernel, FP8 pages
    widened once per workgroup) over FP8 pages at mixed magnitudes, and with V
    growing along units of up to 1024 pages, so that the waves' reference scale
    grows at every 256-page segment while pages are widened one ahead."""
    w = make_workload(3, batch=2, lens=[700, 5000], q_len=96, stale_frac=0.0,
                      kv_mag={"v": ("pages", -3, 4)})
    run_range_case(w, partitions=(0,))
    w = make_workload(3, batch=2, lens=[16384, 4500], q_len=96, stale_frac=0.0,
                      kv_mag={"v": ("ramp", -4, 4)})
    run_range_case(w, partitions=(0, 1))


@pytest.mark.parametrize("D", [128, 64])
def test_head_layout_magnitudes(D):
    lens = np.array([[1, 17, 300, 1500, 4097, 16, 33, 900],
                     [2048, 5, 64, 65, 700, 4096, 1, 250]])
    for mag in ({"v": 1e-4, "k": 1e3}, {"v": ("ramp", -4, 4)}):
        sigma = (1.0 / np.sqrt(D)) / (1e3 if "k" in mag else 1.0)
        w = make_workload(4, lens=lens, kv="fp8", head_dim=D, stale_frac=0.0, kv_mag=mag,
                          sigma=sigma)
        run_range_case(w, partitions=(0, 1, 3))
