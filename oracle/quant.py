"""Dynamic FP8 (e4m3) quantization — oracle (test infrastructure).

Three quantizers, all with the same rule and differing only in the set of
elements that share one scale:

* ``act_quant_block``: one scale per 1x128 block along the last dimension of a
  row-major [M, K] activation ("How to Profile DeepSeek-V3 Inference Kernels
  Using Triton Autotuning", section "Benchmarking the Activation Quantization
  Kernel": ``act_quant(x, block_size=128)`` returns the e4m3 tensor ``y`` and
  the per-block scales ``s``; section "Understanding the Autotuned Kernels in
  DeepSeek-V3": block-wise quantization producing FP8 tensors and per-block
  scaling factors).
* ``amax_quant_tensor``: one scale for the whole tensor, from an exact amax
  over every element (TensorRT-LLM PR "Size the per-tensor FP8 dynamic-quant
  amax grid to the input", sections "Description" and "Correctness": the amax
  is an exact reduction and the scale is amax / 448).
* ``weight_quant_block``: one scale per 128x128 block of a row-major [N, K]
  weight (the block-scaled weights the FP8 GEMM of the DeepSeek-V3 page takes
  as ``b_s``; the same rule applied to square blocks).

The rule for a group G of bf16 values x:
    amax  = max over G of |x|                      (exact)
    s     = fl32(amax / 448)                       (IEEE fp32 division)
    q[i]  = e4m3(clamp(fl32(x[i] / s), -448, 448)) (fp32 division, then RNE)
with the reading that a group with amax = 0 gets s = 0 and all-zero (0x00)
codes, since x / 0 is undefined and every element of such a group is zero.

The power-of-two ("ue8m0") variants (the DeepSeek-V3 page's benchmark of
``act_quant_kernel`` passes ``scale_fmt="ue8m0"``; the page gives no formula)
take, as the plainest reading, the smallest power of two not below amax/448,
so that |x / s| <= 448 still holds and dequantization is exact:
    s     = 2^e,  e = max(ceil(log2(amax / 448)), -127)   (exact; -127 is the
            smallest exponent an unsigned e8m0 scale byte holds)
    q[i]  = e4m3(clamp(fl32(x[i] / s), -448, 448))        (the quotient is exact
            unless it falls below the fp32 normal range, then correctly rounded)
and the same amax = 0 reading (s = 0, codes 0x00).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

F448 = np.float32(448.0)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def _quant_groups(xf: np.ndarray):
    """Quantize a float32 array of shape [G, n]: each row is one group."""
    amax = np.max(np.abs(xf), axis=1)                 # exact
    s = (amax / F448).astype(np.float32)               # IEEE fp32 division
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s)
    y = (xf / safe[:, None]).astype(np.float32)        # IEEE fp32 division
    y = np.clip(y, -F448, F448)
    q = e4m3.encode(y)
    q[zero] = 0                                         # all-zero group
    return q, s


UE8M0_MIN_EXP = -127


def ue8m0_scale(amax: np.ndarray) -> np.ndarray:
    """Smallest power of two s >= amax / 448 (s >= 2^-127); 0 where amax is 0.

    Decided with exact comparisons: amax is a float32 and 448 * 2^e is exact in
    float64, so ``448 * 2^(e-1) < amax <= 448 * 2^e`` fixes e without rounding.
    """
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    pos = a > 0
    _, E = np.frexp(np.where(pos, a / 448.0, 1.0))      # a/448 in [2^(E-1), 2^E), approximately
    e = E.astype(np.int64)
    e = np.where(448.0 * np.ldexp(1.0, e - 1) >= a, e - 1, e)
    e = np.where(448.0 * np.ldexp(1.0, e) < a, e + 1, e)
    e = np.maximum(e, UE8M0_MIN_EXP)
    return np.where(pos, np.ldexp(1.0, e), 0.0).astype(np.float32)


def _quant_groups_ue8m0(xf: np.ndarray):
    """As _quant_groups with the power-of-two scale."""
    amax = np.max(np.abs(xf), axis=1)
    s = ue8m0_scale(amax)
    zero = s == 0
    safe = np.where(zero, np.float32(1.0), s)
    y = (xf / safe[:, None]).astype(np.float32)         # IEEE fp32 division
    y = np.clip(y, -F448, F448)
    q = e4m3.encode(y)
    q[zero] = 0
    return q, s


def act_quant_block(x_bits: np.ndarray, block: int = 128):
    """1x128 block quantization of a bf16 [M, K] tensor.

    Returns ``(q, s)``: ``q`` uint8 e4m3 codes [M, K] and ``s`` float32 scales
    [M, K // block] (block b of row m covers columns b*block .. b*block+block-1).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    xf = bf16_to_f32(x_bits).reshape(M * (K // block), block)
    q, s = _quant_groups(xf)
    return q.reshape(M, K), s.reshape(M, K // block)


def amax_tensor(x_bits: np.ndarray) -> np.float32:
    """Exact amax of a bf16 tensor, as float32."""
    return np.max(np.abs(bf16_to_f32(x_bits)))


def amax_quant_tensor(x_bits: np.ndarray):
    """Per-tensor dynamic quantization of a bf16 tensor of any shape.

    Returns ``(q, s)``: uint8 codes of the same shape and a float32 scalar.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    xf = bf16_to_f32(x_bits).reshape(1, -1)
    q, s = _quant_groups(xf)
    return q.reshape(x_bits.shape), np.float32(s[0])


def static_quant_tensor(x_bits: np.ndarray, scale) -> np.ndarray:
    """Per-tensor quantization of a bf16 tensor with a given scale.

    The apply-only step of the per-tensor quantizer (TensorRT-LLM PR "Size
    the per-tensor FP8 dynamic-quant amax grid to the input", sections
    "Description" and "Correctness": the dynamic op keeps the existing
    quantize-with-a-scale op, whose bytes the dynamic op must reproduce):
        q[i] = e4m3(clamp(fl32(x[i] / s), -448, 448))
    with s the given float32 scale, and, as for a group whose amax is 0, all
    codes 0x00 when s = 0. Scales that are negative or not finite are outside
    the contract. Returns uint8 codes of x's shape.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    s = np.float32(scale)
    if s == 0:
        return np.zeros(x_bits.shape, dtype=np.uint8)
    y = (bf16_to_f32(x_bits) / s).astype(np.float32)   # IEEE fp32 division
    return e4m3.encode(np.clip(y, -F448, F448))


def weight_quant_block(w_bits: np.ndarray, block: int = 128):
    """128x128 block quantization of a bf16 [N, K] weight.

    Returns ``(q, s)``: uint8 codes [N, K] and float32 scales
    [N // block, K // block].
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if N % block or K % block:
        raise ValueError("N and K must be multiples of the block size")
    nb, kb = N // block, K // block
    wf = bf16_to_f32(w_bits).reshape(nb, block, kb, block).transpose(0, 2, 1, 3)
    q, s = _quant_groups(wf.reshape(nb * kb, block * block))
    q = q.reshape(nb, kb, block, block).transpose(0, 2, 1, 3).reshape(N, K)
    return np.ascontiguousarray(q), s.reshape(nb, kb)


def act_quant_block_ue8m0(x_bits: np.ndarray, block: int = 128):
    """1x128 block quantization with power-of-two scales (module docstring).

    Same layout as ``act_quant_block``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    xf = bf16_to_f32(x_bits).reshape(M * (K // block), block)
    q, s = _quant_groups_ue8m0(xf)
    return q.reshape(M, K), s.reshape(M, K // block)


def weight_quant_block_ue8m0(w_bits: np.ndarray, block: int = 128):
    """128x128 block quantization with power-of-two scales (module docstring).

    Same layout as ``weight_quant_block``.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    if N % block or K % block:
        raise ValueError("N and K must be multiples of the block size")
    nb, kb = N // block, K // block
    wf = bf16_to_f32(w_bits).reshape(nb, block, kb, block).transpose(0, 2, 1, 3)
    q, s = _quant_groups_ue8m0(wf.reshape(nb * kb, block * block))
    q = q.reshape(nb, kb, block, block).transpose(0, 2, 1, 3).reshape(N, K)
    return np.ascontiguousarray(q), s.reshape(nb, kb)


def act_quant_block_f32(x: np.ndarray, block: int = 128):
    """1x128 block quantization of a float32 [M, K] tensor (the DeepSeek-V3
    page's ``act_quant`` example quantizes a float32 tensor: section
    "Benchmarking the Activation Quantization Kernel"). Same rule as
    ``act_quant_block`` with the float32 values as they are (finite inputs).
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    M, K = x.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    q, s = _quant_groups(x.reshape(M * (K // block), block))
    return q.reshape(M, K), s.reshape(M, K // block)
