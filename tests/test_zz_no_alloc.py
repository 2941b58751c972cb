"""pa_decode_noalloc on the GPU: the decode with the library's static scratch in
place of a caller's workspace (for callers that cannot allocate device memory).

Checked through the C ABI against pa_decode, the entry point it varies:
outputs and flags bit for bit, on two calls in a row -- the second with a
smaller batch, table and partition count, so it runs over the scratch the
first one left behind -- at several partition counts, with stale tags (flagged
rows); one call is also checked against the fp64 oracle (max-abs 1e-2,
mean-abs 1e-3).  A call that needs more scratch than the library holds is
refused with PA_ERR_SCRATCH before any launch, leaving its output untouched.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload
from tests.oracle_fill import oracle_sequences_parallel
from tests.test_gpu_parity import compare_outputs, log

pytestmark = pytest.mark.gpu

PA_ERR_SCRATCH = -5
SCRATCH_BYTES = 32 << 20


def _pair(dw, parts, rows=None):
    """pa_decode (own workspace) and pa_decode_noalloc on rows [0, rows) of the
    batch: (out, flags) of each."""
    w = dw.w
    n = w.B if rows is None else rows
    bt, lens, q = dw.block_table[:n], dw.lens[:n], dw.q[:n]
    exp = dw.expected_tags[:n]
    f_ref = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    f_na = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    ref = pa.decode(dw.cache, q, bt, lens, w.sigma, expected_tags=exp, flags=f_ref,
                    num_partitions=parts)
    got = pa.decode_noalloc(dw.cache, q, bt, lens, w.sigma, expected_tags=exp, flags=f_na,
                            num_partitions=parts)
    torch.cuda.synchronize()
    return ref, f_ref, got, f_na


@pytest.mark.parametrize("parts", [0, 3, 8])
def test_noalloc_matches_decode_on_two_calls(parts):
    w = make_workload(3, batch=12, lens=[16, 17, 999, 4096, 5000, 16384, 1, 300, 8000, 12000,
                                         64, 2049], stale_frac=0.01)
    dw = build_device_workload(w)
    dw.step_append()
    for rows, p in ((w.B, parts), (5, max(parts - 2, 0))):   # the second call is smaller
        log("noalloc: rows %d partitions %d" % (rows, p))
        ref, f_ref, got, f_na = _pair(dw, p, rows)
        assert torch.equal(f_ref, f_na)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (rows, p)
    if parts == 0:
        fl = f_na.cpu().numpy().view(np.uint32)
        ora = oracle_sequences_parallel(w, range(5), with_pools=False)
        compare_outputs(got, ora, range(5), fl, "noalloc vs oracle")


def test_noalloc_headwise_then_seq():
    """A HEAD-layout cache, then a smaller SEQ one, through the same scratch."""
    lens = np.array([[33, 1, 512, 16, 17, 100, 5, 64], [2048, 8, 4096, 4097, 15, 16, 31, 1000]])
    for w in (make_workload(4, lens=lens, stale_frac=0.02),
              make_workload(2, batch=3, lens=[40, 300, 2000], stale_frac=0.0)):
        dw = build_device_workload(w)
        dw.step_append()
        for p in (0, 16):
            ref, f_ref, got, f_na = _pair(dw, p)
            assert torch.equal(f_ref, f_na)
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (w.layout, p)


def test_noalloc_refuses_calls_beyond_the_scratch():
    """64 sequences x 64 query heads x 64 partitions of fp32 partials need 136 MB."""
    w = make_workload(5, batch=64, lens=[40] * 64, stale_frac=0.0)
    cache = pa.PagedKVCache(w.layout, w.kv_dtype, w.P, w.Hkv, w.D)
    bt = torch.from_numpy(w.block_table).cuda()
    lens = torch.from_numpy(w.lens).cuda()
    q = torch.from_numpy(w.q).view(torch.bfloat16).cuda()
    need = pa.workspace_bytes(cache, bt, lens, w.Hq, num_partitions=64)
    assert need > SCRATCH_BYTES
    out = torch.full(q.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.decode_noalloc(cache, q, bt, lens, w.sigma, num_partitions=64, out=out)
    assert e.value.code == PA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)                     # nothing was launched
    assert "static" in pa.lib().pa_strerror(PA_ERR_SCRATCH).decode()
    # the same call with a workspace runs
    pa.decode(cache, q, bt, lens, w.sigma, num_partitions=64, out=out)
    torch.cuda.synchronize()
