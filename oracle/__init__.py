"""The oracle: a plain, slow, fp64 CPU implementation of the ReplaySSM decode step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import anything in this package. The HIP
library and its Python binding never import it, and it imports nothing from
them: the two sides share no code, tables or constants.

What it computes, and where each piece comes from:

* ``mamba2``  the Mamba-2 decode recurrence (the SSD layer's recurrent form as
  published by Dao and Gu, 2024) and the checkpoint-plus-buffer forms of it.
* ``gdn``     the Gated DeltaNet decode recurrence (gated delta rule as
  published by Yang, Kautz and Hatamizadeh, 2024) and its UT/WY form over a
  buffer of recent inputs.
* ``ring``    the integer state machine of the input buffer: slots, the flush
  schedule, speculative append and commit (sitech.ge ReplaySSM page, sections
  "How ReplaySSM works" and "Reducing state traffic and simplifying rollback").
* ``quant``   the block-scaled 4-bit read copy and the fp16 / fp8 checkpoint
  formats (sitech.ge ReplaySSM page, "Bounding quantization error"), emulated
  exactly in float32.
* ``decode``  drivers that run the method token by token in fp64: conventional
  decode, ReplaySSM decode (checkpoint + buffer), speculative rounds, and the
  snapshot/restore speculative baseline.

Floating point is fp64 except inside the quantizers, whose formats fix fp32
scale arithmetic. Every function states the passage or published definition
it follows; the tests pin each one to something other than itself (brute
force, closed forms, invariants, library routines).
"""
from . import mamba2, gdn, ring, quant, decode  # noqa: F401
