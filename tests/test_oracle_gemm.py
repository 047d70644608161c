"""Pins for the oracle's block-scaled GEMM and its comparison rule (CPU only).

Independent checks:
* unit scales: the float64 reference equals an int64 brute force exactly
  (every e4m3 value is an integer multiple of 2**-9, so products are integer
  multiples of 2**-18 and the sums are exact);
* exact rational brute force in the pages' block form
  sum_b sa[m,b] * sw[n//128,b] * sum_{k in b} A[m,k] W[n,k], with random fp32
  block scales, on shapes with several row and column blocks (M != N != K so
  that a transposed operand or scale fails);
* identity weight: W = I (N = K) and sw = 1 give R = dequantized A;
* the comparison accepts the correctly rounded reference and rejects a result
  with one block scale missing.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3, gemm

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def rand_codes(rng, shape):
    return rng.choice(FINITE, size=shape).astype(np.uint8)


def test_unit_scales_equal_int64_bruteforce():
    rng = np.random.default_rng(1)
    M, N, K = 5, 256, 384
    qa, qw = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    R = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    ia = (e4m3.DECODE[qa] * 2 ** 9).astype(np.int64)
    iw = (e4m3.DECODE[qw] * 2 ** 9).astype(np.int64)
    exact = ia @ iw.T
    assert np.array_equal(R * 2.0 ** 18, exact.astype(np.float64))


def test_fraction_bruteforce_block_form():
    rng = np.random.default_rng(2)
    M, N, K = 3, 256, 384
    qa, qw = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = (10.0 ** rng.uniform(-3, 1, size=(M, K // 128))).astype(np.float32)
    sw = (10.0 ** rng.uniform(-4, -1, size=(N // 128, K // 128))).astype(np.float32)
    R = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    S = gemm.gemm_abs_ref(qa, sa, qw, sw)
    dec = [Fraction(float(v)) if np.isfinite(v) else None for v in e4m3.DECODE]
    cols = [0, 1, 127, 128, 200, 255]
    for m in range(M):
        for n in cols:
            tot, atot = Fraction(0), Fraction(0)
            for b in range(K // 128):
                part, apart = Fraction(0), Fraction(0)
                for k in range(b * 128, (b + 1) * 128):
                    p = dec[qa[m, k]] * dec[qw[n, k]]
                    part += p
                    apart += abs(p)
                scale = Fraction(float(sa[m, b])) * Fraction(float(sw[n // 128, b]))
                tot += scale * part
                atot += scale * apart
            # float64 reference within one rounding per product sum of |terms|
            assert abs(Fraction(float(R[m, n])) - tot) <= atot * Fraction(K + 2, 2 ** 53)
            assert abs(Fraction(float(S[m, n])) - atot) <= atot * Fraction(K + 2, 2 ** 53)


def test_identity_weight():
    rng = np.random.default_rng(3)
    M, K = 7, 256
    qa = rand_codes(rng, (M, K))
    sa = (10.0 ** rng.uniform(-2, 2, size=(M, K // 128))).astype(np.float32)
    qw = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qw, 0x38)                      # 1.0
    sw = np.ones((K // 128, K // 128), np.float32)
    R = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    Abar = e4m3.DECODE[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    assert np.array_equal(R, Abar)


def test_scale_indexing_is_per_block():
    # one activation block scale and one weight block scale doubled: only the
    # matching (row, K block) and (column block, K block) terms change
    rng = np.random.default_rng(4)
    M, N, K = 4, 384, 256
    qa, qw = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    base = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    sa2 = sa.copy(); sa2[2, 1] = 2.0
    d = gemm.gemm_blockscaled_ref(qa, sa2, qw, sw) - base
    blk = (e4m3.DECODE[qa[2, 128:]] @ e4m3.DECODE[qw[:, 128:]].T)
    assert np.array_equal(d[2], blk) and not d[[0, 1, 3]].any()
    sw2 = sw.copy(); sw2[1, 0] = 4.0
    d = gemm.gemm_blockscaled_ref(qa, sa, qw, sw2) - base
    blk = 3.0 * (e4m3.DECODE[qa[:, :128]] @ e4m3.DECODE[qw[128:256, :128]].T)
    assert np.array_equal(d[:, 128:256], blk)
    assert not d[:, :128].any() and not d[:, 256:].any()


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(200_000).astype(np.float32) * np.float32(1000.0)
    v = np.concatenate([v, np.float32([0.0, -0.0, 1.00390625, 1.01171875, 3e38, 1e-40])])
    ours = gemm.f64_to_bf16_rne(v.astype(np.float64))
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def normal_codes(rng, shape, scale):
    """e4m3 codes of N(0, scale) values (what quantized activations look like)."""
    v = np.clip(rng.standard_normal(shape) * scale, -448, 448).astype(np.float32)
    return e4m3.encode(v)


@pytest.mark.parametrize("chained", [False, True])
def test_compare_accepts_reference_and_rejects_wrong_results(chained):
    rng = np.random.default_rng(6)
    M, N, K = 8, 256, 512
    qa, qw = normal_codes(rng, (M, K), 100.0), normal_codes(rng, (N, K), 100.0)
    sa = (10.0 ** rng.uniform(-2, 0, size=(M, K // 128))).astype(np.float32)
    sw = (10.0 ** rng.uniform(-3, -1, size=(N // 128, K // 128))).astype(np.float32)
    R = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    S = gemm.gemm_abs_ref(qa, sa, qw, sw)
    Se = gemm.gemm_exp_envelope_ref(qa, sa, qw, sw)
    good = gemm.f64_to_bf16_rne(R)
    cmp = lambda c: gemm.compare_gemm(c, R, S, K, Se, chained=chained)
    res = cmp(good)
    assert res["ok"], res
    # one activation block scale lost
    sa_bad = sa.copy(); sa_bad[:, 2] = 1.0
    bad = gemm.f64_to_bf16_rne(gemm.gemm_blockscaled_ref(qa, sa_bad, qw, sw))
    assert not cmp(bad)["ok"]
    # transposed weight blocks
    bad = gemm.f64_to_bf16_rne(gemm.gemm_blockscaled_ref(qa, sa, qw, sw[::-1]))
    assert not cmp(bad)["ok"]
    # one K block dropped
    qa_bad = qa.copy(); qa_bad[:, 128:256] = 0
    bad = gemm.f64_to_bf16_rne(gemm.gemm_blockscaled_ref(qa_bad, sa, qw, sw))
    assert not cmp(bad)["ok"]
    # a result off by 2**-6 relative everywhere
    bad = gemm.f64_to_bf16_rne(R * (1 + 2.0 ** -6))
    assert not cmp(bad)["ok"]
    # a power-of-two scale off by one exponent in one block
    sw_bad = sw.copy(); sw_bad[0, 1] *= 2
    bad = gemm.f64_to_bf16_rne(gemm.gemm_blockscaled_ref(qa, sa, qw, sw_bad))
    assert not cmp(bad)["ok"]


def test_exp_envelope_closed_form():
    codes = np.arange(256, dtype=np.uint8)
    env = gemm.exp_envelope(codes)
    d = np.abs(e4m3.DECODE)
    fin = np.isfinite(d)
    normal = fin & (((codes >> 3) & 0xF) > 0)
    # normal values: 2**e <= |v| < 2**(e+1)
    assert np.all(env[normal] <= d[normal]) and np.all(d[normal] < 2 * env[normal])
    # subnormals: envelope 2**-6 above the value; zeros: 0
    sub = fin & (((codes >> 3) & 0xF) == 0) & ((codes & 0x7) != 0)
    assert np.all(env[sub] == 2.0 ** -6) and np.all(d[sub] < 2.0 ** -6)
    assert env[0x00] == 0 and env[0x80] == 0
    assert env[0x7E] == 256.0 and env[0x38] == 1.0


def test_tensorscaled_ref_is_block_ref_with_constant_blocks():
    rng = np.random.default_rng(51)
    M, N, K = 9, 256, 384
    qa, qw = normal_codes(rng, (M, K), 50.0), normal_codes(rng, (N, K), 50.0)
    sa, sw = np.float32(0.0371), np.float32(2.5e-4)
    R1 = gemm.gemm_tensorscaled_ref(qa, sa, qw, sw)
    R2 = gemm.gemm_blockscaled_ref(qa, np.full((M, K // 128), sa, np.float32), qw,
                                   np.full((N // 128, K // 128), sw, np.float32))
    S1 = gemm.gemm_tensorscaled_abs_ref(qa, sa, qw, sw)
    # the two differ only by float64 rounding (the block path rounds each
    # product of dequantized values, up to 56 bits wide)
    assert np.all(np.abs(R1 - R2) <= 1e-13 * S1)
    assert np.all(S1 >= np.abs(R1))
    # a lost scale is far outside that
    assert not np.all(np.abs(R1 / float(sw) - R2) <= 1e-13 * S1)


def test_tensorscaled_ref_integer_bruteforce():
    # integer-valued codes and power-of-two scales: exact in int64
    rng = np.random.default_rng(52)
    ints = np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0xB8, 0xC0, 0x00], np.uint8)   # 1,2,3,4,5,-1,-2,0
    qa = rng.choice(ints, (4, 256)); qw = rng.choice(ints, (128, 256))
    A = e4m3.DECODE[qa].astype(np.int64); W = e4m3.DECODE[qw].astype(np.int64)
    want = (A @ W.T).astype(np.float64) * 0.25 * 8.0
    assert np.array_equal(gemm.gemm_tensorscaled_ref(qa, np.float32(0.25), qw, np.float32(8.0)), want)
