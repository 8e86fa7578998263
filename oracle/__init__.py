"""CPU oracle for the SageAttention2 quantized attention forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg are the only code allowed to import this package.  The GPU library and its Python
binding never import or call it, and it imports nothing from them.

Modules:
  fp8   -- OCP FP8 E4M3 codec (RNE, saturating), written from the format's definition.
  sage  -- the method step by step (exact means, smoothing, grouped quantization, Delta_S,
           integer QK^T, online softmax with FP8 P~ and V, two-level accumulation) and
           exact fp64 attention for accuracy reporting.
  range_study -- the (P_r, V_r) narrowing study of an fp16 P~V accumulator (oracle only).
"""
from . import fp8, sage  # noqa: F401
from .sage import (DEFAULT, Geometry, Prologue, attend_block, delta_s, exact_attention,  # noqa: F401
                   exact_mean, prologue, sage_attention, scores_int)
