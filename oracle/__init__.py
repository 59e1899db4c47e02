"""CPU oracle for exact scaled-dot-product attention (float64, numpy).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU path.  `attention` is the plain
definition (materialised S and P); `tile_model` is a CPU model of the blocked
online-softmax algorithm used to check its recurrence against the definition.
"""
from .attention import (scores, softmax_rows, forward, forward_rows, backward,  # noqa: F401
                        decode, merge_partials, backward_cross)
