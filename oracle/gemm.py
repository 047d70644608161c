"""Block-scaled FP8 GEMM — fp64 oracle and comparison rules (test infrastructure).

What the GEMM computes ("How to Profile DeepSeek-V3 Inference Kernels Using
Triton Autotuning", sections "Understanding the Autotuned Kernels in
DeepSeek-V3" and "Benchmarking the FP8 GEMM Kernel": a matmul of e4m3 matrices
with per-block scaling factors ``a_s`` and ``b_s``, K tiled by 128):

    C[m, n] = sum_b  sa[m, b] * sw[n // 128, b] * sum_{k in block b} A[m, k] * W[n, k]

with A [M, K] e4m3 and sa [M, K/128] (1x128 activation blocks), W [N, K] e4m3
and sw [N/128, K/128] (128x128 weight blocks), C = A . W^T of shape [M, N] and
bf16 output. Because every scale is constant over its block, this equals the
plain product of the dequantized operands, which is what the oracle computes,
in float64: Abar = dec(A) * sa, Wbar = dec(W) * sw, R = Abar @ Wbar^T.

Comparison (a reading; the pages give no GEMM tolerance): the bf16 result C
must satisfy
  (i)  normwise: max|C - R| / max|R| <= 1e-2, and
  (ii) elementwise: |C - R| <= 4 * ulp_bf16(R) + floor, where the floor is
       the accumulation error the specified arithmetic is allowed:
       floor = TAU_MATRIX * Se + tau(K) * S.
S = |Abar| @ |Wbar|^T. tau(K) = (K/128 + 2) * 2**-24 + 2**-20. Its first part
covers the fp32 steps outside the matrix cores: the rounding of each block's
scale product sa*sw and the K/128 rounded adds of scaled block sums into the
fp32 accumulator, in any summation order (Higham, "Accuracy and Stability of
Numerical Algorithms", ch. 4: a sum of n terms loses at most (n-1) u of the
sum of their magnitudes); 2**-20 * S covers, with TAU_MATRIX's 2**-19 * Se,
the matrix cores' 24-bit combining steps inside a block (below). The
128-term dot product of one K block runs on the FP8 matrix cores, which do not
sum at fp32 precision: each run of 8 products is summed in block floating
point, every product aligned to the run's largest input-exponent sum
(e_a + e_w, subnormals counted at exponent -6) with 13 fraction bits and
truncated; runs are then combined at 24 fraction bits. Each run therefore
loses less than 8 * 2**(E_run - 13) <= 2**-10 * sum over the run of
2**(e_a + e_w), and TAU_MATRIX = 2**-10 + 2**-19 with
Se = sum_k (2**e_a * sa) * (2**e_w * sw) (the power-of-two envelope of the
dequantized operands, ``gemm_exp_envelope_ref``) bounds it, the 2**-19 term
covering the 24-bit combining steps. Without the floor no kernel that
accumulates in finite precision can meet 4 ulp where cancellation makes |R|
much smaller than S.

When the matrix cores also apply the (power-of-two) block scales and carry
the fp32 accumulator from one K block to the next as their own accumulator
input, the add of each block into that accumulator is not one rounded fp32
add: each of the up to 8 run-pair sums of a block is added with truncation at
2**(exponent of the accumulator - 24) (measured: eight products of 2**-26 in
eight separate runs vanish next to an accumulator of 1.0), so a block can lose
up to 8 * 2**(e_acc - 24) < 2**-20 * |acc| <= 2**-20 * S. For that path the
accumulation term is tau_chained(K) = (K/128 + 1) * 2**-20 in place of tau(K).
"""
from __future__ import annotations

import numpy as np

from . import e4m3

BLOCK = 128
TAU_MATRIX = 2.0 ** -10 + 2.0 ** -19   # FP8 matrix-core accumulation floor (module docstring)


def dequant_act(qa: np.ndarray, sa: np.ndarray) -> np.ndarray:
    """dec(A) * sa over 1x128 blocks, float64 [M, K] (each product is exact)."""
    qa = np.asarray(qa, dtype=np.uint8)
    M, K = qa.shape
    sa = np.asarray(sa, dtype=np.float32).astype(np.float64)
    if sa.shape != (M, K // BLOCK):
        raise ValueError("activation scale shape must be [M, K/128]")
    return e4m3.decode(qa) * np.repeat(sa, BLOCK, axis=1)


def dequant_weight(qw: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """dec(W) * sw over 128x128 blocks, float64 [N, K] (each product is exact)."""
    qw = np.asarray(qw, dtype=np.uint8)
    N, K = qw.shape
    sw = np.asarray(sw, dtype=np.float32).astype(np.float64)
    if sw.shape != (N // BLOCK, K // BLOCK):
        raise ValueError("weight scale shape must be [N/128, K/128]")
    full = np.repeat(np.repeat(sw, BLOCK, axis=0), BLOCK, axis=1)
    return e4m3.decode(qw) * full


def gemm_blockscaled_ref(qa, sa, qw, sw) -> np.ndarray:
    """Reference C = Abar @ Wbar^T in float64, shape [M, N]."""
    return dequant_act(qa, sa) @ dequant_weight(qw, sw).T


def gemm_abs_ref(qa, sa, qw, sw) -> np.ndarray:
    """S = |Abar| @ |Wbar|^T in float64, the scale of the summation error."""
    return np.abs(dequant_act(qa, sa)) @ np.abs(dequant_weight(qw, sw)).T


def exp_envelope(codes: np.ndarray) -> np.ndarray:
    """2**e of each e4m3 code's exponent field e (subnormals at 2**-6), 0 for
    the zero codes: the alignment magnitude the matrix cores use."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = np.maximum((c >> 3) & 0xF, 1) - 7
    return np.where((c & 0x7F) == 0, 0.0, np.ldexp(1.0, e))


def gemm_exp_envelope_ref(qa, sa, qw, sw) -> np.ndarray:
    """Se = envelope(A) * sa @ (envelope(W) * sw)^T, float64 [M, N]."""
    qa = np.asarray(qa, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    ea = exp_envelope(qa) * np.repeat(np.asarray(sa, np.float32).astype(np.float64), BLOCK, axis=1)
    sw64 = np.asarray(sw, np.float32).astype(np.float64)
    ew = exp_envelope(qw) * np.repeat(np.repeat(sw64, BLOCK, axis=0), BLOCK, axis=1)
    return ea @ ew.T


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, one rounding to nearest, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    mant, expo = np.frexp(v)
    out = np.where(np.abs(v) >= 2.0 ** -126,
                   np.ldexp(np.rint(mant * 256.0), expo - 8),
                   np.rint(v * 2.0 ** 133) * 2.0 ** -133)
    return (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def ulp_bf16(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |r|: 2**(floor(log2|r|) - 7), at least the
    subnormal spacing 2**-133 (which is also the spacing at 0)."""
    r = np.abs(np.asarray(r, dtype=np.float64))
    _, fe = np.frexp(r)
    u = np.ldexp(1.0, fe - 1 - 7)
    # frexp(0) has exponent 0: zero gets the subnormal spacing like any value
    # below 2**-126
    return np.where(r == 0.0, 2.0 ** -133, np.maximum(u, 2.0 ** -133))


def gemm_tolerance_tau(K: int) -> float:
    return (K // BLOCK + 2) * 2.0 ** -24 + 2.0 ** -20


def gemm_tolerance_tau_chained(K: int) -> float:
    """Accumulation term when the matrix cores carry the accumulator over the
    K blocks (module docstring)."""
    return (K // BLOCK + 1) * 2.0 ** -20


def s13_tau(K: int) -> float:
    """The fp32-accumulation floor first proposed for this comparison:
    (128 + K/128 + 2) * 2**-24, i.e. every add of the 128-term block sums, the
    K/128 block adds and the two scale multiplies counted as one fp32
    rounding (Higham, ch. 4). The FP8 matrix cores do not sum a block at fp32
    precision (module docstring), so the comparison uses the wider floor; this
    one is reported beside it, as the share of outputs that meet plain
    4 ulp + this floor."""
    return (BLOCK + K // BLOCK + 2) * 2.0 ** -24


def compare_gemm(c_bits: np.ndarray, R: np.ndarray, S: np.ndarray, K: int, Se: np.ndarray,
                 chained: bool = False):
    """Check a bf16 GEMM result against the fp64 reference.

    Returns a dict with the normwise error, the worst elementwise ratio
    |C-R| / (4 ulp + TAU_MATRIX Se + tau S), a boolean ``ok``; ``chained``
    selects tau_chained (matrix cores carrying the accumulator over K blocks).
    Also: ``frac_plain``, the share of outputs within 4 ulp + s13_tau(K) * S,
    and the pieces ``merge_compare`` needs to combine results over row
    chunks (``max_err``, ``max_abs_ref``, ``n``, ``n_plain``).
    """
    C = bf16_bits_to_f64(c_bits)
    R = np.asarray(R, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    Se = np.asarray(Se, dtype=np.float64)
    err = np.abs(C - R)
    tau = gemm_tolerance_tau_chained(K) if chained else gemm_tolerance_tau(K)
    ulp4 = 4.0 * ulp_bf16(R)
    bound = ulp4 + TAU_MATRIX * Se + tau * S
    part = dict(max_err=float(np.max(err, initial=0.0)),
                max_abs_ref=float(np.max(np.abs(R), initial=0.0)),
                elem_ratio=float(np.max(err / bound, initial=0.0)),
                n=int(err.size),
                n_plain=int(np.count_nonzero(err <= ulp4 + s13_tau(K) * S)))
    return merge_compare([part])


def merge_compare(parts):
    """Combine compare_gemm results over disjoint pieces of one output."""
    max_err = max(p["max_err"] for p in parts)
    rmax = max(p["max_abs_ref"] for p in parts)
    ratio = max(p["elem_ratio"] for p in parts)
    n = sum(p["n"] for p in parts)
    n_plain = sum(p["n_plain"] for p in parts)
    normwise = max_err / rmax if rmax > 0 else max_err
    return dict(normwise=normwise, elem_ratio=ratio, max_err=max_err, max_abs_ref=rmax, n=n,
                n_plain=n_plain, frac_plain=n_plain / n if n else 1.0,
                ok=bool(normwise <= 1e-2 and ratio <= 1.0))


def compare_gemm_full(c_bits, qa, sa, qw, sw, chained=False, per_tensor=False, rows=2048):
    """compare_gemm over the whole output, one block of ``rows`` output rows
    at a time (the reference of each block computed from its rows of A, so
    that large outputs need not hold R, S and Se whole). ``per_tensor``: sa
    and sw are one scale each (the per-tensor-scaled GEMM's reference)."""
    qa = np.asarray(qa, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    c_bits = np.asarray(c_bits, dtype=np.uint16)
    M, K = qa.shape
    N = qw.shape[0]
    if c_bits.shape != (M, N):
        raise ValueError("output shape must be [M, N]")
    if per_tensor:
        sa_blk = np.full((M, K // BLOCK), np.float32(sa), np.float32)
        sw_blk = np.full((N // BLOCK, K // BLOCK), np.float32(sw), np.float32)
    else:
        sa_blk, sw_blk = np.asarray(sa, np.float32), np.asarray(sw, np.float32)
    parts = []
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        a, s = qa[r0:r1], sa_blk[r0:r1]
        if per_tensor:
            R = gemm_tensorscaled_ref(a, sa, qw, sw)
            S = gemm_tensorscaled_abs_ref(a, sa, qw, sw)
        else:
            R = gemm_blockscaled_ref(a, s, qw, sw_blk)
            S = gemm_abs_ref(a, s, qw, sw_blk)
        Se = gemm_exp_envelope_ref(a, s, qw, sw_blk)
        parts.append(compare_gemm(c_bits[r0:r1], R, S, K, Se, chained=chained))
    return merge_compare(parts)


def gemm_tensorscaled_ref(qa, sa, qw, sw):
    """C = sa * sw * (dec(A) . dec(W)^T) in float64, for one scale per tensor
    (the per-tensor dynamic quantization's output feeding the projection GEMM:
    TensorRT-LLM PR "Size the per-tensor FP8 dynamic-quant amax grid to the
    input", section "Description": the quantize step runs ahead of the GEMM and
    hands it the quantized input and the scale). sa and sw are scalars."""
    A = e4m3.DECODE[np.asarray(qa)].astype(np.float64)
    W = e4m3.DECODE[np.asarray(qw)].astype(np.float64)
    return float(np.float32(sa)) * float(np.float32(sw)) * (A @ W.T)


def gemm_tensorscaled_abs_ref(qa, sa, qw, sw):
    A = np.abs(e4m3.DECODE[np.asarray(qa)].astype(np.float64))
    W = np.abs(e4m3.DECODE[np.asarray(qw)].astype(np.float64))
    return abs(float(np.float32(sa)) * float(np.float32(sw))) * (A @ W.T)
