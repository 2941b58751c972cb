"""A decode step captured as a HIP graph replays to the eager result (GPU)."""
import numpy as np
import pytest
import torch

from decode_attention_paged_pa_amd import pa
from decode_attention_paged_pa_amd.device_inputs import build_device_workload
from decode_attention_paged_pa_amd.workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,kw,parts", [(3, dict(batch=4, lens=[100, 2000, 4097, 9000]), 4),
                                          (4, dict(batch=2), 0), (1, {}, 0)])
def test_graph_replays_match_eager(cfg, kw, parts):
    w = make_workload(cfg, stale_frac=0.0, **kw)
    dw = build_device_workload(w)
    dw.step_append()
    eager = dw.decode(check=True, num_partitions=parts).clone()
    eager_flags = dw.flags.clone()
    g = pa.DecodeStepGraph(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step, dw.v_step,
                           dw.q, dw.lens, w.sigma, expected_tags=dw.expected_tags, flags=dw.flags,
                           num_partitions=parts)
    for i in range(4):
        dw.flags.fill_(-1)
        out = g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        assert torch.equal(dw.flags, eager_flags), i
        # eager work between replays (the graph must not depend on it)
        _ = dw.decode(check=False, num_partitions=parts)
        torch.cuda.synchronize()


def test_graph_sees_updated_inputs():
    w = make_workload(2, batch=3, lens=[50, 600, 1500], stale_frac=0.0)
    dw = build_device_workload(w)
    dw.step_append()
    g = pa.DecodeStepGraph(dw.cache, dw.block_table, dw.lens_old, dw.n_step, dw.k_step, dw.v_step,
                           dw.q, dw.lens, w.sigma, expected_tags=dw.expected_tags, flags=dw.flags)
    a = g.replay().clone()
    dw.q.mul_(-1)                      # new queries, written in place
    b = g.replay().clone()
    ref = dw.decode(check=True)
    torch.cuda.synchronize()
    assert not torch.equal(a, b)
    assert torch.equal(b.view(torch.int16), ref.view(torch.int16))
    # a stale tag written in place is caught on the next replay
    dw.expected_tags[1, 0] ^= 1
    out = g.replay()
    torch.cuda.synchronize()
    assert dw.flags.cpu().numpy().view(np.uint32).tolist() == [0, 1, 0]
    assert torch.all(out[1].view(torch.int16) == 0)
