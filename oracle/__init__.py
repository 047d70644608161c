"""CPU oracle for the FP8 quantize-and-multiply path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code that states what the path computes.
It exists to check the HIP library and is not part of the product: only the
test-suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it. It shares no code with the HIP library, and the
library never calls it (there is no CPU fallback).

Modules
-------
``e4m3``  the OCP e4m3 ("fn") format: decode table and round-to-nearest-even
          encoder, from the bit layout (1 sign, 4 exponent, 3 mantissa bits).
``quant`` 1x128 block dynamic activation quantization, the per-tensor variant
          (and its apply step with a given scale) and the 128x128 weight
          block quantization.
``gemm``  the fp64 reference of the block-scaled GEMM over dequantized
          operands, and the comparison rules used against the HIP output.

Every function is pinned by CPU tests (closed forms, invariants, brute force
and library cross-checks) under ``tests/``.
"""
from . import e4m3, quant, gemm  # noqa: F401
