"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE.

Only tests/, the smoke check in __graft_entry__.py and the CPU-baseline leg of
bench.py may import this package.  The product (the HIP library and its Python
binding) never does, and shares no code with it.

Modules:
  codecs -- BF16 and OCP e4m3 conversions written from the format definitions.
  paged  -- append (with FP8 quantisation), tag validation and decode attention
            in fp64, following the pages' description of the paged KV cache,
            the per-head block table, the FP8 KV cache and the integrity check.

Pins (tests/test_oracle_*.py) tie every function to something other than
itself: exhaustive or brute-force codec checks, a library conversion,
closed forms of attention, dense non-paged attention, page-permutation
invariance, brute force at 50 digits on tiny shapes, the split/merge identity,
the scale invariant of the FP8 cache, and the FP8 codes and scales bit for bit
against a rebuild from exact rationals (one rounding to binary32 per named
step, then the nearest e4m3 code by search).  No function here is "parity
unpinned".
"""
from .codecs import (  # noqa: F401
    E4M3_MAX,
    E4M3_VALUES,
    bf16_from_f32_rne,
    bf16_to_f64,
    e4m3_from_f32_rne_sat,
    e4m3_to_f64,
)
from .paged import (  # noqa: F401
    FLAG_LEN_OVERFLOW,
    FLAG_PAGE_OOB,
    FLAG_TAG_MISMATCH,
    OracleCache,
    attention_f64,
    gather_unit,
    lse_merge,
    lse_partial,
    oracle_append,
    oracle_attention_mass,
    oracle_compact,
    oracle_decode,
    oracle_decode_multi,
    oracle_decode_row,
    oracle_score_update,
    oracle_validate,
    units,
)
