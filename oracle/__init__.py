"""CPU oracle for RecSA tree attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never imports it and must fail loudly when its native library is
missing; nothing here is a fallback.
"""
from .recsa import (  # noqa: F401
    INT32_MAX,
    TreeCache,
    UnitResult,
    attend_unit,
    bf16_round,
    build_slice,
    decode,
    dense_unit,
    from_storage,
    generate,
    inv_freq,
    level_counts,
    plan_counts,
    prefill,
    rope_rows,
    rope_table,
    rotate,
    round_store,
    to_storage,
)
