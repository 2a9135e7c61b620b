"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This package only draws random numbers and lays them out; it contains none of
the attention arithmetic. Both the CPU oracle (``oracle/``) and the HIP
library are fed from here and from nowhere else.
"""

from .synth import (  # noqa: F401
    CHUNK_ROWS,
    Workload,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    c3_prefill_block,
    make_multi_query,
    make_workload,
    static_window_ranges,
)
