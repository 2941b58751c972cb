"""Page runs at the edges of the attention kernels' page-loop structure, on a GPU.

The page loops walk a unit's pages in segments (their ids loaded and waited for
once: 256 pages for FP8 caches, 512 for BF16 with one or two column tiles, 128
for BF16 with four) and, inside a segment, in 64-page chunks with one id
register each: the loop's last iteration in a chunk reads its look-ahead page
ids from the next chunk's register.  These lengths end just before, at and just
after the chunk and segment edges (some with a partial last page), so that with
one partition a unit's run ends at each of them, and with the automatic split
the runs start past them.  Every kernel kind: one query (FP8, BF16), 4 drafts
(two column tiles), 8 drafts (four tiles, FP8 and BF16) and a prefill chunk
(the page-sharing kernel, BF16 and FP8).  Bars as in the other parity tests.
"""
import pytest

from decode_attention_paged_pa_amd.workloads import make_workload
from tests.test_gpu_parity import run_case

pytestmark = pytest.mark.gpu

# tokens: 63, 64, 65, 67, 128, 129, 256, 257, 513 and 1025 pages
EDGE_LENS = [63 * 16, 64 * 16, 64 * 16 + 1, 67 * 16 - 3, 128 * 16, 128 * 16 + 7,
             256 * 16, 257 * 16 - 1, 513 * 16 - 9, 1025 * 16 - 2]
WIDTH = 1040   # table entries: room for the longest


@pytest.mark.parametrize("cfg,q_len,kw", [
    (3, 1, dict(stale_frac=0.0)),                 # FP8, one query: 256-page segments
    (2, 1, dict()),                               # BF16, one query: 512-page segments
    (5, 4, dict()),                               # FP8, 4 drafts x G 8: two tiles
    (5, 8, dict()),                               # FP8, 8 drafts x G 8: four tiles, one K buffer
    (2, 8, dict(heads=(64, 8))),                  # BF16, four tiles: 128-page segments
])
def test_runs_at_chunk_and_segment_edges(cfg, q_len, kw):
    w = make_workload(cfg, batch=len(EDGE_LENS), lens=EDGE_LENS, q_len=q_len, table_width=WIDTH, **kw)
    run_case(w, partitions=(1, 0))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_runs_at_chunk_and_segment_edges(kv):
    """The page-sharing kernel (128-token chunk of G 4: 512 columns, 16 blocks):
    its ring requests run 3 pages ahead (BF16) or 2 pages ahead of the page
    each wave widens, one page ahead of the one computed (FP8), and cross the
    same edges."""
    lens = EDGE_LENS[:8] + [513 * 16 - 9]
    w = make_workload(2, batch=len(lens), lens=lens, q_len=128, table_width=WIDTH, kv=kv)
    run_case(w, partitions=(1, 0))
