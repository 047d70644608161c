"""Pins for the oracle's block, per-tensor and weight quantizers (CPU only).

Independent checks:
* exact rational brute force (fractions.Fraction): the scale is the binary32
  value nearest to amax/448 and each code is the e4m3 value nearest to the
  binary32 value nearest to x/s, found by search over all codes;
* an exhaustive grid over every (bf16 significand of the block maximum,
  bf16 significand of an element) pair, checked against a float64-division
  computation (a double-precision quotient of two binary32 values rounded once
  to binary32 is the correctly rounded binary32 quotient, since 53 >= 2*24+2),
  and shown to catch the plausible mistake of multiplying by a reciprocal;
* invariants: amax is the largest |x|, the element(s) at amax encode to +-448,
  every code is within half an e4m3 step of the clamped quotient, zero blocks
  give scale 0 and zero codes;
* known answers: blocks of e4m3 values times 2**j with maximum 448 * 2**j have
  scale exactly 2**j and reproduce their own codes.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import e4m3, quant

F448 = np.float32(448.0)


# --------------------------------------------------------------------------
# exact helpers written for the tests (no oracle code)

def fl32(r: Fraction) -> Fraction:
    """Round a rational to binary32, nearest with ties to even (no overflow)."""
    if r == 0:
        return Fraction(0)
    neg = r < 0
    r = -r if neg else r
    e = r.numerator.bit_length() - r.denominator.bit_length()
    while Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = r / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * quantum
    return -out if neg else out


POS_CODES = [(c, Fraction(float(e4m3.DECODE[c]))) for c in range(0x7F)]


def nearest_e4m3(y: Fraction, negative: bool) -> int:
    a = min(abs(y), Fraction(448))
    best = None
    for c, v in POS_CODES:
        d = abs(v - a)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0] | (0x80 if negative else 0)


def bf16_value(bits) -> Fraction:
    return Fraction(float(quant.bf16_to_f32(np.array([bits], np.uint16))[0]))


def brute_group(bits_list):
    """Scale and codes of one group by exact arithmetic."""
    vals = [bf16_value(b) for b in bits_list]
    amax = max(abs(v) for v in vals)
    s = fl32(amax / 448)
    if s == 0:
        return 0.0, [0] * len(vals)
    codes = []
    for b, v in zip(bits_list, vals):
        y = fl32(v / s)
        codes.append(nearest_e4m3(y, negative=bool(int(b) & 0x8000)))
    return float(s), codes


def nearest_code_vec(v32):
    """Vectorised nearest search (same rule as nearest_e4m3)."""
    pos = e4m3.DECODE[:0x7F]
    a = np.minimum(np.abs(v32.astype(np.float64)), 448.0)
    i = np.searchsorted(pos, a, side="left")
    hi = np.clip(i, 0, 0x7E)
    lo = np.clip(i - 1, 0, 0x7E)
    dlo, dhi = a - pos[lo], pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    return np.where(pick_hi, hi, lo).astype(np.uint8) | (np.signbit(v32).astype(np.uint8) << 7)


def widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------

def test_block_quant_fraction_bruteforce():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 256)) * np.array([[1.0], [1e-3], [50.0]])
    x[1, 5] = 7e3                      # one outlier block
    x[2, 128:] = 0.0                   # one zero block
    bits = synth.f64_to_bf16_bits(x)
    q, s = quant.act_quant_block(bits)
    assert q.shape == (3, 256) and s.shape == (3, 2) and s.dtype == np.float32
    for m in range(3):
        for b in range(2):
            es, ec = brute_group(list(bits[m, b * 128:(b + 1) * 128]))
            assert float(s[m, b]) == es, (m, b)
            assert list(q[m, b * 128:(b + 1) * 128]) == ec, (m, b)


def test_special_blocks_fraction_bruteforce():
    blocks = synth.special_blocks()
    q, s = quant.act_quant_block(blocks)
    for i in range(blocks.shape[0]):
        es, ec = brute_group(list(blocks[i]))
        assert float(s[i, 0]) == es, i
        assert list(q[i]) == ec, i


def test_quotient_grid_exhaustive():
    g = synth.quotient_grid()
    q, s = quant.act_quant_block(g)
    xf = widen(g)
    amax = np.max(np.abs(xf), axis=1)
    s_ref = (amax.astype(np.float64) / 448.0).astype(np.float32)
    assert np.array_equal(s[:, 0].view(np.uint32), s_ref.view(np.uint32))
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xf.astype(np.float64) / s_ref.astype(np.float64)[:, None]).astype(np.float32)
    q_ref = nearest_code_vec(y)
    q_ref[s_ref == 0] = 0
    assert np.array_equal(q, q_ref)
    # the grid is sharp enough to reject a reciprocal multiply in place of x/s
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (np.float32(1.0) / s_ref).astype(np.float32)
        y_bad = (xf * r[:, None]).astype(np.float32)
    q_bad = nearest_code_vec(y_bad)
    assert np.count_nonzero(q_bad != q_ref) > 0


def test_amax_invariants():
    rng = np.random.default_rng(3)
    bits = synth.f64_to_bf16_bits(rng.standard_t(3.0, size=(5, 384)))
    vals = [float(v) for v in widen(bits).reshape(-1)]
    amax = quant.amax_tensor(bits)
    assert float(amax) == max(abs(v) for v in vals)
    perm = rng.permutation(bits.size)
    assert quant.amax_tensor(bits.reshape(-1)[perm]) == amax
    # per block: the scale times 448 brackets the block maximum
    _, s = quant.act_quant_block(bits)
    for m in range(5):
        for b in range(3):
            blk = vals[m * 384 + b * 128: m * 384 + (b + 1) * 128]
            bm = max(abs(v) for v in blk)
            assert float(s[m, b]) == float(fl32(Fraction(bm) / 448))


def test_max_element_encodes_to_448_and_half_step():
    bits = synth.gen_c1()["a"]
    q, s = quant.act_quant_block(bits)
    xf = widen(bits).reshape(-1, 128)
    qb = q.reshape(-1, 128)
    sb = s.reshape(-1)
    zero = sb == 0
    assert np.all(qb[zero] == 0) and zero.sum() == 1
    amax = np.max(np.abs(xf), axis=1)
    at_max = (np.abs(xf) == amax[:, None]) & ~zero[:, None]
    assert np.all((qb[at_max] & 0x7F) == 0x7E)
    # every code within half an e4m3 step of the clamped binary32 quotient
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.clip((xf / sb[:, None]).astype(np.float32), -F448, F448)[~zero].astype(np.float64)
    d = e4m3.decode(qb[~zero])
    a = np.abs(y)
    gap = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(d - y) <= gap / 2)


def test_known_answer_power_of_two_scales():
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    rows, want_q, want_s = [], [], []
    for j in range(-8, 8):
        codes = rng.choice(finite, size=128)
        codes[rng.integers(0, 128)] = 0x7E if j % 2 else 0xFE
        codes[np.abs(e4m3.DECODE[codes]) == 448] = 0x7E if j % 2 else 0xFE
        vals = e4m3.DECODE[codes] * 2.0 ** j
        rows.append(synth.f64_to_bf16_bits(vals))
        want_q.append(codes)
        want_s.append(2.0 ** j)
    bits = np.stack(rows).reshape(-1, 256)             # two blocks per row
    q, s = quant.act_quant_block(bits)
    assert np.array_equal(q.reshape(-1, 128), np.stack(want_q).astype(np.uint8))
    assert np.array_equal(s.reshape(-1), np.array(want_s, np.float32))


def test_block_axis_and_shape():
    # rows of very different magnitude: blocks run along K within one row
    M, K = 4, 512
    x = np.ones((M, K)) * np.array([[1.0], [2.0], [4.0], [8.0]])
    x[:, 128:256] *= 1000.0
    q, s = quant.act_quant_block(synth.f64_to_bf16_bits(x))
    for m in range(M):
        for b in range(K // 128):
            assert s[m, b] == np.float32(x[m, b * 128] / 448.0)
    assert np.all((q & 0x7F) == 0x7E)
    with pytest.raises(ValueError):
        quant.act_quant_block(np.zeros((2, 100), np.uint16))


def test_per_tensor_rules():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 128))
    x[2, 17] = -300.0                                  # the tensor maximum
    bits = synth.f64_to_bf16_bits(x)
    q, s = quant.amax_quant_tensor(bits)
    es, ec = brute_group(list(bits.reshape(-1)))
    assert float(s) == es
    assert list(q.reshape(-1)) == ec
    assert q.shape == bits.shape
    # one 1x128 block: per-tensor and block quantization agree
    q1, s1 = quant.amax_quant_tensor(bits[:1])
    qb, sb = quant.act_quant_block(bits[:1])
    assert np.array_equal(q1, qb) and s1 == sb[0, 0]
    # all zeros
    qz, sz = quant.amax_quant_tensor(np.full((2, 64), 0x8000, np.uint16))
    assert sz == 0 and np.all(qz == 0)


def test_weight_quant_block_rules():
    rng = np.random.default_rng(13)
    N, K = 256, 384                                    # N != K: catches transposed blocks
    w = rng.standard_normal((N, K)) * 0.02
    mult = 2.0 ** rng.integers(-6, 7, size=(N // 128, K // 128))
    w *= np.repeat(np.repeat(mult, 128, axis=0), 128, axis=1)
    bits = synth.f64_to_bf16_bits(w)
    q, s = quant.weight_quant_block(bits)
    assert q.shape == (N, K) and s.shape == (N // 128, K // 128)
    for i in range(N // 128):
        for j in range(K // 128):
            blk = bits[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qq, ss = quant.amax_quant_tensor(blk)
            assert s[i, j] == ss
            assert np.array_equal(q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128], qq)
    # spot-check one block against exact arithmetic
    blk = bits[128:256, 256:384].reshape(-1)
    es, ec = brute_group(list(blk[:1]) + list(blk))   # same max set
    amax = max(abs(bf16_value(b)) for b in blk)
    assert float(s[1, 2]) == float(fl32(amax / 448))


# --------------------------------------------------------------------------
# power-of-two ("ue8m0") scales

def exact_pow2_scale(amax: Fraction) -> Fraction:
    """Smallest 2^e >= amax/448 with e >= -127, by exact search (0 for amax 0)."""
    if amax == 0:
        return Fraction(0)
    e = -127
    while Fraction(2) ** e * 448 < amax:
        e += 1
    return Fraction(2) ** e


def test_ue8m0_scale_exhaustive_over_bf16():
    # every positive finite bf16 value as the amax, against exact search
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    got = quant.ue8m0_scale(widen(bits))
    step = 97   # the exact search is slow in Python: every 97th pattern plus the extremes
    for b in list(range(1, 0x7F80, step)) + [1, 2, 0x7F7F, 0x7F7E, 0x0080, 0x007F]:
        want = exact_pow2_scale(bf16_value(b))
        assert Fraction(float(got[b - 1])) == want, (hex(b), got[b - 1], want)
    # every result is a power of two, not below amax/448, and its half is below
    a = widen(bits).astype(np.float64)
    s = got.astype(np.float64)
    m, _ = np.frexp(s)
    assert np.all(m == 0.5)
    assert np.all(s * 448.0 >= a)
    clamped = s == 2.0 ** -127
    assert np.all((s / 2 * 448.0 < a) | clamped)


def test_ue8m0_scale_closed_forms():
    for k in range(-120, 120):
        a = np.float32(448.0 * 2.0 ** k)
        assert quant.ue8m0_scale(np.array([a]))[0] == np.float32(2.0 ** k), k
        up = np.float32(a * (1 + 2.0 ** -7))           # the next bf16 value up
        assert quant.ue8m0_scale(np.array([up]))[0] == np.float32(2.0 ** (k + 1)), k
        down = np.float32(a * (1 - 2.0 ** -8))         # the next bf16 value down (1.75 -> 1.7421875)
        assert quant.ue8m0_scale(np.array([down]))[0] == np.float32(2.0 ** k), k
    assert quant.ue8m0_scale(np.array([np.float32(0.0)]))[0] == 0.0
    assert quant.ue8m0_scale(np.array([np.float32(1e-38)]))[0] == np.float32(2.0 ** -127)


def test_ue8m0_block_quant_properties():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    bits = synth.f64_to_bf16_bits(x)
    bits[3, 128:256] = 0                            # zero block
    q, s = quant.act_quant_block_ue8m0(bits)
    xf = widen(bits).reshape(64, 4, 128).astype(np.float64)
    sd = s.astype(np.float64)
    assert s[3, 1] == 0 and not q[3, 128:256].any()
    nz = sd > 0
    m, _ = np.frexp(sd[nz])
    assert np.all(m == 0.5)
    # codes are the nearest e4m3 (ties to even) of the exact quotient x / s
    y = np.where(nz[..., None], xf / np.where(nz, sd, 1.0)[..., None], 0.0)
    assert np.all(np.abs(y) <= 448.0)
    want = nearest_code_vec(y.astype(np.float32).reshape(64, 512))
    want[3, 128:256] = 0
    assert np.array_equal(q, want)
    # the block's largest code lies in (224, 448] (scale within a factor 2 of amax/448)
    dec = np.abs(e4m3.DECODE[q].reshape(64, 4, 128))
    assert np.all(dec.max(axis=2)[nz] > 224.0 * (1 - 2.0 ** -4))


def test_ue8m0_fraction_bruteforce():
    rng = np.random.default_rng(12)
    for t in range(6):
        bits = synth.f64_to_bf16_bits(rng.standard_normal(128) * 10.0 ** rng.uniform(-30, 30))
        q, s = quant.act_quant_block_ue8m0(bits.reshape(1, 128))
        vals = [bf16_value(b) for b in bits]
        sw = exact_pow2_scale(max(abs(v) for v in vals))
        assert Fraction(float(s[0, 0])) == sw
        for i, (b, v) in enumerate(zip(bits, vals)):
            assert q[0, i] == nearest_e4m3(fl32(v / sw), negative=bool(int(b) & 0x8000)), (t, i)


def test_ue8m0_matches_fp32_rule_when_scale_is_power_of_two():
    # amax / 448 a power of two: both rules give the same scale and codes
    rng = np.random.default_rng(13)
    x = rng.uniform(-1, 1, (16, 256))
    x[:, 0] = 448.0 * 2.0 ** rng.integers(-30, 30, 16)     # the amax of block 0
    x[:, 128] = -3.5 * 2.0 ** rng.integers(-30, 30, 16)     # and of block 1 (3.5 = 448 / 128)
    x[:, 1:128] *= np.abs(x[:, :1]) / 2
    x[:, 129:] *= np.abs(x[:, 128:129]) / 2
    bits = synth.f64_to_bf16_bits(x)
    q1, s1 = quant.act_quant_block(bits)
    q2, s2 = quant.act_quant_block_ue8m0(bits)
    assert np.array_equal(s1, s2) and np.array_equal(q1, q2)


def test_ue8m0_weight_blocks():
    rng = np.random.default_rng(14)
    w = synth.f64_to_bf16_bits(rng.standard_normal((256, 384)) * 0.02)
    q, s = quant.weight_quant_block_ue8m0(w)
    assert q.shape == (256, 384) and s.shape == (2, 3)
    for bn in range(2):
        for bk in range(3):
            blk = w[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            qb, sb = quant.act_quant_block_ue8m0(blk.reshape(1, -1), block=128 * 128)
            assert sb[0, 0] == s[bn, bk]
            assert np.array_equal(qb.reshape(128, 128), q[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128])



# --------------------------------------------------------------------------
# float32 input

def brute_group_f32(vals32):
    vals = [Fraction(float(v)) for v in vals32]
    amax = max(abs(v) for v in vals)
    s = fl32(amax / 448)
    if s == 0:
        return 0.0, [0] * len(vals)
    return float(s), [nearest_e4m3(fl32(v / s), negative=bool(np.signbit(v32)))
                      for v, v32 in zip(vals, vals32)]


def test_f32_input_fraction_bruteforce():
    rng = np.random.default_rng(31)
    for t in range(5):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-35, 35)).astype(np.float32)
        x[3] = -x[3]
        q, s = quant.act_quant_block_f32(x.reshape(1, 128))
        sw, codes = brute_group_f32(x)
        assert float(s[0, 0]) == sw
        assert list(q[0]) == codes, t


def test_f32_input_reduces_to_bf16_rule_on_bf16_values():
    # float32 values that are bf16 values quantize exactly as the bf16 path
    bits = synth.gen_c1()["a"]
    q1, s1 = quant.act_quant_block(bits)
    q2, s2 = quant.act_quant_block_f32(widen(bits))
    assert np.array_equal(q1, q2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_f32_input_full_precision_matters():
    # values with more than 8 significant bits: the quotient uses all of them
    x = np.full((1, 128), np.float32(1.0), np.float32)
    x[0, 0] = np.float32(448.0)                       # amax -> scale exactly 1.0
    x[0, 1] = np.float32(1.0625 + 2.0 ** -20)         # just above the tie 1.0625 (between 1.0 and 1.125)
    x[0, 2] = np.float32(1.0625)                      # the tie itself: to even (1.0, code 0x38)
    q, s = quant.act_quant_block_f32(x)
    assert s[0, 0] == 1.0
    assert q[0, 1] == 0x39 and q[0, 2] == 0x38


# --------------------------------------------------------------------------
# per-tensor quantization with a given (static) scale

def test_static_quant_fraction_bruteforce():
    # exact rationals: each code is the e4m3 value nearest to the binary32
    # value nearest to x / s, for scales that are not of the form amax/448,
    # including one below 2^-64 and quotients that saturate or underflow
    rng = np.random.default_rng(21)
    x = rng.standard_normal(96) * np.logspace(-6, 3, 96)
    x[::7] *= -1
    x[5] = 0.0
    bits = synth.f64_to_bf16_bits(x)
    bits[6] = 0x8000                                    # -0 keeps its sign
    for s in (np.float32(0.0123), np.float32(1.0), np.float32(3.0e-3), np.float32(2.5),
              np.float32(7.0e-21), np.float32(6.1e-5)):
        q = quant.static_quant_tensor(bits, s)
        assert q.dtype == np.uint8 and q.shape == bits.shape
        sf = Fraction(float(s))
        want = [nearest_e4m3(fl32(bf16_value(b) / sf), negative=bool(int(b) & 0x8000)) for b in bits]
        assert list(q) == want, float(s)


def test_static_quant_reproduces_dynamic_codes():
    # given the dynamic scale, the static op returns the dynamic op's bytes
    # (the correctness statement of the per-tensor page)
    for seed, shape, mult in ((3, (4, 2048), 1.0), (4, (1, 2048), 1e-4), (5, (7, 130), 3e2)):
        x = np.random.default_rng(seed).standard_normal(shape) * mult
        bits = synth.f64_to_bf16_bits(x)
        q, s = quant.amax_quant_tensor(bits)
        assert np.array_equal(quant.static_quant_tensor(bits, s), q)
    zero = np.zeros((3, 64), np.uint16)
    q, s = quant.amax_quant_tensor(zero)
    assert s == 0 and np.array_equal(quant.static_quant_tensor(zero, s), q)


def test_static_quant_known_answers():
    # e4m3 grid values times 2^j quantized with s = 2^j give back their own
    # codes; past 448 * s the codes saturate to +-448; a zero scale gives 0x00
    j = -5
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = e4m3.DECODE[codes].astype(np.float64) * 2.0 ** j
    bits = synth.f64_to_bf16_bits(vals)
    assert np.array_equal(widen(bits).astype(np.float64), vals)   # exact in bf16
    q = quant.static_quant_tensor(bits, np.float32(2.0 ** j))
    want = codes.copy()
    want[codes == 0x80] = 0x80
    assert np.array_equal(q, want)
    big = synth.f64_to_bf16_bits(np.array([1e3, -1e3, 449.0, -460.0, 1e-9, -1e-9]))
    assert list(quant.static_quant_tensor(big, np.float32(1.0))) == [0x7E, 0xFE, 0x7E, 0xFE, 0x00, 0x80]
    assert np.all(quant.static_quant_tensor(big, np.float32(0.0)) == 0)


def test_static_quant_near_e4m3_midpoints():
    # scales for which x / s lands within a few binary32 steps of a midpoint
    # between two e4m3 values: there the binary32 rounding of the quotient
    # decides the code (multiplying by a rounded reciprocal, or rounding the
    # exact quotient straight to e4m3, gives a different code in some cases).
    # Reference: the binary32 quotient from a float64 division (correctly
    # rounded, 53 >= 2*24 + 2), then the nearest search over the code table.
    xb = np.arange(0x3F80, 0x4000, dtype=np.uint16)            # bf16 in [1, 2)
    xb = np.concatenate([xb, xb | 0x8000])
    xf = widen(xb).astype(np.float64)
    pos = e4m3.DECODE[:0x7F].astype(np.float64)
    mids = (pos[0x30:0x48] + pos[0x31:0x49]) / 2
    rng = np.random.default_rng(23)
    checked = 0
    for x0 in rng.choice(xf[:128], 24, replace=False):
        for t in mids:
            s0 = np.float32(x0 / t)
            for k in range(-2, 3):
                s = s0
                for _ in range(abs(k)):
                    s = np.nextafter(s, np.float32(np.inf if k > 0 else 0), dtype=np.float32)
                q = quant.static_quant_tensor(xb, s)
                y = (xf / np.float64(s)).astype(np.float32)
                want = nearest_code_vec(np.clip(y, -F448, F448))
                assert np.array_equal(q, want), (float(x0), float(t), k)
                checked += 1
    assert checked == 24 * len(mids) * 5
