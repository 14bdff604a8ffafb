"""CPU oracle for the MoE decode/verify layer step (test infrastructure).

A slow, plain float64 NumPy implementation of what the GPU library computes,
written from the pages' description of the method.  It is test infrastructure:
only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it.  It shares no code with the GPU library and never imports it; the two meet
only through the seeded input generator, which holds none of the method's
arithmetic.
"""
from . import formats, layer  # noqa: F401
from .layer import (attention_block, expert_ffn, layer_step, route,  # noqa: F401
                    score_shift, stack_step, window_bounds)
