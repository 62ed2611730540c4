"""CPU fp64 oracle of the triangle multiplicative update (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path never calls it and shares no code with it.
"""

from .trimul_oracle import (  # noqa: F401
    bf16_round,
    bf16_bits_to_f64,
    layer_norm,
    sigmoid,
    forward,
    forward_block,
    Intermediates,
)
