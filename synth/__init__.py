"""Seeded synthetic inputs for the CSA indexer score / top-k path.

This package holds none of the indexer's arithmetic.  It only draws queries,
compressed keys, head weights, segment ids and decode positions with the shapes
and value distributions of the indexer workloads, and rounds them to bfloat16
bit patterns.  Both sides of every parity test (the CPU oracle and the HIP
library) and the benchmark take their inputs from here.
"""

from .inputs import (  # noqa: F401
    CONFIG_TITLES,
    CONFIGS,
    Problem,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_config,
    make_problem,
)
