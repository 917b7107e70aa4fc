"""Seeded synthetic inputs for the verify step.

This package draws random inputs and encodes them (bf16 rounding, page
tables); it holds none of the verify method's arithmetic.  Both the CPU
oracle's tests and the HIP path's tests and bench take their inputs from
here, so the two sides always see the same bits.
"""

from .gen import (bf16_bits, bf16_to_f32, uniforms24, make_reject_inputs,  # noqa: F401
                  make_attn_inputs, kv_layout_x)
from .configs import CONFIGS, get_config, SIGMA_FOR_ALPHA  # noqa: F401
