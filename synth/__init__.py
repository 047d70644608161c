"""Seeded synthetic inputs for the FP8 quantize-and-multiply path.

This module only draws random numbers and rounds them to the storage type of
the inputs (bf16, or fp32 for drawn scales). It holds none of the path's own
arithmetic (no amax, no scale, no e4m3 rounding, no matmul), so the CPU oracle
under ``oracle/`` and the HIP library can both be fed from it without sharing
any code with each other.

Every generator is deterministic: the stream for configuration ``cfg``, row
count ``M`` and operand ``stream`` (0 = activation A or X, 1 = weight W,
2 = drawn weight scales) is ``numpy.random.default_rng([cfg, M, stream])``.

The workloads follow the quantize-and-multiply path of DeepSeek-style FP8
inference ("How to Profile DeepSeek-V3 Inference Kernels Using Triton
Autotuning", sections "Benchmarking the FP8 GEMM Kernel" and "Benchmarking the
Activation Quantization Kernel") and the per-tensor sweep of TensorRT-LLM PR
"Size the per-tensor FP8 dynamic-quant amax grid to the input" (section "Test
Coverage", K=2048 with M from 1 to 65536).

bf16 values are returned as ``numpy.uint16`` bit patterns (row-major).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "CONFIGS",
    "rng_for",
    "f64_to_bf16_bits",
    "bf16_bits_to_f64",
    "normal_bf16",
    "gen_c1",
    "gen_c2",
    "gen_c3",
    "gen_c4",
    "gen_c5",
    "gen_config",
    "quotient_grid",
    "special_blocks",
]

# Shapes of the five workloads. W always arrives as bf16 and is block-quantized
# (128x128) by the caller before the GEMM.
CONFIGS = {
    1: dict(name="tiny block quant + GEMM", M=[32], N=512, K=512),
    2: dict(name="per-tensor dynamic quant sweep", M=[1, 64, 256, 1024, 65536], K=2048),
    3: dict(name="decode block-scaled GEMM", M=[1, 8, 32, 64], N=2048, K=7168),
    4: dict(name="prefill block-scaled GEMM", M=[4096], N=4096, K=7168),
    5: dict(name="large-M stress", M=[16384], N=7168, K=2048),
}


def rng_for(cfg: int, M: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg), int(M), int(stream)])


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values once, to nearest with ties to even, to bf16 bits.

    Finite inputs of magnitude below the bf16 maximum only (the generators
    never produce anything else).
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    mant, expo = np.frexp(v)  # v = mant * 2**expo, 0.5 <= |mant| < 1
    normal = np.abs(v) >= 2.0 ** -126
    # 8 significant bits in the normal range: rint(mant * 2**8) * 2**(expo - 8)
    out[normal] = np.ldexp(np.rint(mant[normal] * 256.0), expo[normal] - 8)
    # fixed spacing 2**-133 below 2**-126
    sub = ~normal
    out[sub] = np.rint(v[sub] * 2.0 ** 133) * 2.0 ** -133
    if not np.all(np.isfinite(out)) or np.any(np.abs(out) > 3.3895313892515355e38):
        raise ValueError("value outside the finite bf16 range")
    return (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64 (for generator checks)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def normal_bf16(shape, std: float, rng: np.random.Generator) -> np.ndarray:
    return f64_to_bf16_bits(rng.standard_normal(size=shape) * std)


def gen_c1(M: int = 32, K: int = 512, N: int = 512):
    """Tiny case: A ~ N(0,1) with 1% of entries multiplied by 50 and one
    all-zero 1x128 block; W ~ N(0, 0.02), to be block-quantized 128x128."""
    rng = rng_for(1, M, 0)
    a = rng.standard_normal(size=(M, K))
    n_out = int(round(0.01 * M * K))
    idx = rng.choice(M * K, size=n_out, replace=False)
    a.reshape(-1)[idx] *= 50.0
    zb = int(rng.integers(0, M * (K // 128)))
    a.reshape(-1, 128)[zb] = 0.0
    w = rng_for(1, M, 1).standard_normal(size=(N, K)) * 0.02
    return dict(a=f64_to_bf16_bits(a), w=f64_to_bf16_bits(w), zero_block=zb)


def gen_c2(M: int, K: int = 2048):
    """Per-tensor sweep: X ~ N(0,1), shape [M, K]."""
    return dict(x=normal_bf16((M, K), 1.0, rng_for(2, M, 0)))


def gen_c3(M: int, K: int = 7168, N: int = 2048):
    """Decode: A ~ N(0,1) with a seeded 1% of entries replaced by
    Student-t(nu=3) draws; W ~ N(0, 0.02), to be block-quantized 128x128."""
    rng = rng_for(3, M, 0)
    a = rng.standard_normal(size=(M, K))
    n_out = max(1, int(round(0.01 * M * K)))
    idx = rng.choice(M * K, size=n_out, replace=False)
    a.reshape(-1)[idx] = rng.standard_t(3.0, size=n_out)
    w = rng_for(3, M, 1).standard_normal(size=(N, K)) * 0.02
    return dict(a=f64_to_bf16_bits(a), w=f64_to_bf16_bits(w))


def gen_c4(M: int = 4096, K: int = 7168, N: int = 4096):
    """Prefill: A ~ N(0,1); W ~ N(0, 0.02), to be block-quantized 128x128."""
    a = normal_bf16((M, K), 1.0, rng_for(4, M, 0))
    w = normal_bf16((N, K), 0.02, rng_for(4, M, 1))
    return dict(a=a, w=w)


def gen_c5(M: int = 16384, K: int = 2048, N: int = 7168):
    """Large-M stress: A ~ Student-t(nu=3); 0.1% of the 1x128 blocks set to
    +0; another, disjoint 0.1% each get one element of magnitude >= 1e4
    (10**U[4,5], random sign). W ~ N(0, 0.02) is block-quantized 128x128 and
    its scales are then replaced by log-uniform draws in [1e-4, 1e-1]."""
    rng = rng_for(5, M, 0)
    a = rng.standard_t(3.0, size=(M, K))
    nblk = M * (K // 128)
    n_sp = max(1, int(round(0.001 * nblk)))
    blocks = rng.choice(nblk, size=2 * n_sp, replace=False)
    zero_blocks, big_blocks = blocks[:n_sp], blocks[n_sp:]
    ab = a.reshape(-1, 128)
    ab[zero_blocks] = 0.0
    pos = rng.integers(0, 128, size=n_sp)
    mag = 10.0 ** rng.uniform(4.0, 5.0, size=n_sp)
    sign = np.where(rng.integers(0, 2, size=n_sp) == 1, -1.0, 1.0)
    ab[big_blocks, pos] = sign * mag
    a_bits = f64_to_bf16_bits(a)
    # bf16 rounding may pull a value just under 1e4: move it to the next bf16 up
    flat = a_bits.reshape(-1, 128)
    for b, p in zip(big_blocks, pos):
        while abs(bf16_bits_to_f64(flat[b, p])) < 1e4:
            flat[b, p] = np.uint16(int(flat[b, p]) + 1)
    w = rng_for(5, M, 1).standard_normal(size=(N, K)) * 0.02
    rs = rng_for(5, M, 2)
    sw = (10.0 ** rs.uniform(-4.0, -1.0, size=(N // 128, K // 128))).astype(np.float32)
    return dict(a=a_bits, w=f64_to_bf16_bits(w), w_scale=sw,
                zero_blocks=np.sort(zero_blocks), big_blocks=np.sort(big_blocks))


def gen_config(cfg: int, M: int | None = None):
    """Dispatch by configuration number (1..5)."""
    if cfg == 1:
        return gen_c1()
    if cfg == 2:
        return gen_c2(M)
    if cfg == 3:
        return gen_c3(M)
    if cfg == 4:
        return gen_c4()
    if cfg == 5:
        return gen_c5()
    raise ValueError(f"unknown configuration {cfg}")


def quotient_grid(amax_exponents=(0, -20, 20, -100, -118, -126, 100)):
    """Blocks of 128 bf16 values that cover, for each amax exponent given, every
    pair (bf16 significand of the block maximum, bf16 significand of an
    element), with elements from the block maximum's binade down to 14
    binades below it, of both signs.

    Row layout: element 0 of every block holds the block maximum (+ or -),
    elements 1..127 hold other values no larger in magnitude. Returns bf16 bits
    [n_blocks, 128]. No random numbers: the grid is exhaustive by design.
    """
    rows = []
    for ae in amax_exponents:
        for am in range(128):                     # significand of the maximum
            amax_bits = ((127 + ae) << 7) | am    # positive bf16 of the max
            vals = []
            for de in range(0, 15):               # binades below the maximum
                e = 127 + ae - de
                if e < 1:
                    continue
                for m in range(128):
                    b = (e << 7) | m
                    if b > amax_bits:
                        continue
                    vals.append(b)
                    vals.append(b | 0x8000)
            vals = np.array(vals, dtype=np.uint16)
            for i in range(0, len(vals), 127):
                chunk = vals[i:i + 127]
                blk = np.zeros(128, dtype=np.uint16)
                blk[0] = amax_bits if (i // 127) % 2 == 0 else (amax_bits | 0x8000)
                blk[1:1 + len(chunk)] = chunk
                # pad a short last chunk with copies (never above the maximum)
                if len(chunk) < 127:
                    blk[1 + len(chunk):] = chunk[0]
                rows.append(blk)
    return np.stack(rows)


def special_blocks():
    """Hand-made 1x128 blocks for edge cases, bf16 bits [n, 128]: all +0, all
    -0, mixed signed zeros, one nonzero among zeros, constant blocks, a single
    huge value over tiny ones, the bf16 extremes (largest finite, smallest
    subnormal) and values at e4m3 rounding ties when the scale is 1."""
    def b(vals):
        return f64_to_bf16_bits(np.asarray(vals, dtype=np.float64))
    blocks = []
    blocks.append(np.zeros(128, np.uint16))                           # +0
    blocks.append(np.full(128, 0x8000, np.uint16))                    # -0
    z = np.zeros(128, np.uint16); z[::2] = 0x8000; blocks.append(z)   # +-0
    one = np.zeros(128, np.uint16); one[77] = b([-3.5])[0]; blocks.append(one)
    blocks.append(b(np.full(128, 0.1)))                               # constant
    blocks.append(b(np.full(128, -7.0e3)))
    huge = b(-np.linspace(1e-3, 1e-2, 128)); huge[5] = b([6.0e4])[0]; blocks.append(huge)
    ext = np.full(128, 0x0001, np.uint16); ext[0] = 0x7F7F; blocks.append(ext)  # max, min sub
    ext2 = np.full(128, 0x8001, np.uint16); ext2[9] = 0xFF7F; blocks.append(ext2)
    tiny = np.full(128, 0x0080, np.uint16); tiny[3] = 0x0081; blocks.append(tiny)  # 2^-126 range
    # scale exactly 1 (block maximum 448): ties of the e4m3 grid in every binade
    ties = [448.0]
    ties += [(m + 0.5) * 2.0 ** -9 for m in range(8)]          # subnormal ties
    for e in range(-6, 8):                                       # normal ties
        for m in range(8):
            ties.append(2.0 ** e * (1 + m / 8.0) + 2.0 ** (e - 4))
    ties = np.array(ties + [0.0] * (128 - len(ties)))
    tb = b(ties)
    blocks.append(tb)
    tb2 = tb.copy(); tb2[1:] |= 0x8000; blocks.append(tb2)
    return np.stack(blocks)
