"""OCP e4m3 ("fn") format: decode table and encoder (oracle; test infrastructure).

Format, as described on the page "Converting DeepSeek-V4's Indexer GEMM from
FP32 to bf16" (section "Assumptions and Their Validity", assumption 1): one sign
bit, four exponent bits, three mantissa bits; every e4m3 value widens to bf16
without loss. The largest finite magnitude is 448, the divisor of the dynamic
scale on the TensorRT-LLM page "Size the per-tensor FP8 dynamic-quant amax grid
to the input" (section "Correctness": scale = amax / 448). This is the "fn"
variant (``float8_e4m3fn``, named in "How to Profile DeepSeek-V3 Inference
Kernels Using Triton Autotuning", section "Benchmarking the FP8 GEMM Kernel"):
exponent bias 7, no infinities, S.1111.111 is NaN, subnormals at exponent
field 0.

Readings where the pages are silent:
* rounding is to nearest with ties to even;
* values are clamped to [-448, 448] before rounding (saturation), so nothing
  encodes to NaN;
* the sign is kept for values that round to zero (-tiny -> 0x80).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9


def decode_table() -> np.ndarray:
    """Value of each of the 256 codes as float64 (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = (code >> 7) & 1
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
            continue
        if e == 0:
            mag = 2.0 ** -6 * (m / 8.0)           # subnormal
        else:
            mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)  # normal
        vals[code] = -mag if s else mag
    return vals


DECODE = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(v: np.ndarray) -> np.ndarray:
    """Round float32 values to e4m3 codes: clamp to +-448, then round to the
    nearest e4m3 value, ties to even; the sign bit of ``v`` is kept.

    Work is in float64, where every step below is exact for float32 input.
    NaN input is outside the contract.
    """
    v32 = np.asarray(v, dtype=np.float32)
    sign = ((v32.view(np.uint32) >> 31).astype(np.uint8)) << 7
    a = np.minimum(np.abs(v32.astype(np.float64)), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)

    normal = a >= MIN_NORMAL
    an = a[normal]
    _, fe = np.frexp(an)            # an = f * 2**fe, 0.5 <= f < 1
    e = fe - 1                      # floor(log2(an))
    r = np.rint(an * np.exp2(3 - e))  # 8 <= r <= 16, ties to even
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    code[normal] = ((e + 7) << 3) | (r.astype(np.int64) - 8)

    sub = ~normal
    # below 2**-6 the spacing is 2**-9; r == 8 lands on the smallest normal
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    return (code.astype(np.uint8) | sign).astype(np.uint8)
