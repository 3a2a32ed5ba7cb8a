"""Seeded synthetic inputs for the int4 weight-streaming decode path.

This package is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds only the input recipe (shapes, seeded draws, the offline
int4 quantiser that turns N(0, 0.02) weights into packed codes plus scales, and
bf16 rounding of drawn values); it holds none of the decode arithmetic.
"""

from .shapes import SHAPES, ModelShape  # noqa: F401
from .inputs import (  # noqa: F401
    TENSOR_IDS,
    bf16_bits,
    bf16_value,
    make_embedding,
    make_hidden,
    make_kv,
    make_layer,
    make_lm_head,
    make_x,
    quantize_int4,
    rng_for,
)
