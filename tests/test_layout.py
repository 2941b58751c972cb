"""The pool read-back helper (decode_attention_paged_pa_amd/layout.py) on the CPU.

pool_to_logical reads the documented block order back with a reshape and a
transpose; it must equal indexing with the element maps k_offsets /
v_offsets and the V slot map, for every cache format (and odd pool sizes,
where the last page's V stays in its own slot)."""
import numpy as np
import pytest

from decode_attention_paged_pa_amd.layout import pool_to_logical, pool_to_logical_by_index


@pytest.mark.parametrize("layout,kv,D,H,P", [
    ("seq", "fp8", 128, 8, 7), ("seq", "bf16", 128, 8, 6), ("seq", "fp8", 64, 3, 5),
    ("seq", "bf16", 64, 1, 9), ("seq", "fp8", 128, 1, 4), ("head", "fp8", 128, 8, 11),
    ("head", "bf16", 128, 8, 10), ("head", "fp8", 64, 2, 3), ("head", "bf16", 64, 4, 1)])
def test_fast_read_back_equals_the_index_maps(layout, kv, D, H, P):
    e = 1 if kv == "fp8" else 2
    heads = H if layout == "seq" else 1
    raw = np.random.default_rng(P * D + H).integers(0, 256, size=P * heads * 16 * D * e,
                                                     dtype=np.uint8)
    for which in ("k", "v"):
        a = pool_to_logical(raw, which, layout, kv, P, H, D)
        b = pool_to_logical_by_index(raw, which, layout, kv, P, H, D)
        assert a.shape == b.shape == (P, heads, 16, D)
        assert np.array_equal(a, b), (which, layout, kv, D, H, P)
