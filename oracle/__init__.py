"""CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library never does.
"""
from .oracle import (Oracle, rms_norm, rope, rope_cos_sin, sigmoid, silu, softmax_rows,
                     gqa_attention, linear, greedy_argmax, greedy_argmax_fast,
                     top_k, top2_gap, param_count, tensor_count)
from . import sampling
from . import generate
from . import quant
