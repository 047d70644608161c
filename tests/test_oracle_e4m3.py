"""Pins for the oracle's e4m3 decode table and encoder (CPU only).

The encoder is checked against things other than itself:
* hand-derived cases (tests/golden/e4m3_hand_cases.txt),
* an independent nearest-value search over the decode table with ties to
  even, exhaustively over every float32 whose magnitude lies in
  [2**-12, 2**10) (all rounding decisions of the format happen there) and on
  every bf16 bit pattern,
* torch's CPU float8_e4m3fn conversion (clamped first, since torch turns
  overflow into NaN rather than saturating).
"""
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_cases.txt")


def nearest_code(v32: np.ndarray) -> np.ndarray:
    """Independent encoder: nearest finite e4m3 magnitude by table search,
    ties broken toward the code with an even last mantissa bit."""
    v32 = np.asarray(v32, dtype=np.float32)
    pos = e4m3.DECODE[:0x7F]                 # codes 0x00..0x7E, increasing
    a = np.minimum(np.abs(v32.astype(np.float64)), 448.0)
    i = np.searchsorted(pos, a, side="left")
    hi = np.clip(i, 0, 0x7E)
    lo = np.clip(i - 1, 0, 0x7E)
    dlo = a - pos[lo]
    dhi = pos[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(v32).astype(np.uint8)) << 7
    return code | sign


def torch_code(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.clip(np.asarray(v32, dtype=np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_constants():
    d = e4m3.DECODE
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x08] == 2.0 ** -6
    assert d[0x01] == 2.0 ** -9
    assert d[0x38] == 1.0
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    nan = np.isnan(d)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_decode_monotone_and_symmetric():
    pos = e4m3.DECODE[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert len(np.unique(pos)) == 127
    assert np.array_equal(e4m3.DECODE[0x80:0xFF], -pos)


def test_decode_exact_in_bf16():
    # every e4m3 value widens to bf16 (and so to fp32) without loss
    fin = e4m3.DECODE[np.isfinite(e4m3.DECODE)]
    f32 = fin.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), fin)
    trunc = (f32.view(np.uint32) & 0xFFFF0000).view(np.float32)
    assert np.array_equal(trunc, f32)


def test_decode_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (t == e4m3.DECODE) | (np.isnan(t) & np.isnan(e4m3.DECODE))
    assert same.all()


def _golden_cases():
    vals, codes = [], []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals.append(float(parts[0]))
            codes.append(int(parts[1], 16))
    return np.array(vals, dtype=np.float32), np.array(codes, dtype=np.uint8)


def test_encode_hand_cases():
    v, c = _golden_cases()
    assert len(v) >= 20
    got = e4m3.encode(v)
    bad = [(float(x), hex(g), hex(e)) for x, g, e in zip(v, got, c) if g != e]
    assert not bad, bad


def test_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.DECODE[codes].astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_encode_all_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    got = e4m3.encode(v)
    assert np.array_equal(got, nearest_code(v))
    assert np.array_equal(got, torch_code(v))


def test_encode_exhaustive_rounding_range():
    # every positive float32 in [2**-12, 2**10): all ties, carries, the
    # subnormal/normal boundary and the saturation point lie in here
    lo = (127 - 12) << 23
    hi = (127 + 10) << 23
    step = 1 << 24
    for start in range(lo, hi, step):
        bits = np.arange(start, min(start + step, hi), dtype=np.uint32)
        v = bits.view(np.float32)
        got = e4m3.encode(v)
        assert np.array_equal(got, nearest_code(v)), hex(start)
        assert np.array_equal(got, torch_code(v)), hex(start)


def test_encode_sign_symmetry_and_far_ranges():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    got = e4m3.encode(v)
    assert np.array_equal(got, nearest_code(v))
    assert np.array_equal(got, torch_code(v))
    # the sign bit only toggles bit 7
    assert np.array_equal(e4m3.encode(-v) ^ got, np.full(got.shape, 0x80, np.uint8))
    tiny = np.array([2.0 ** -12, 2.0 ** -40, 1e-45, -1e-45, -2.0 ** -11], np.float32)
    assert list(e4m3.encode(tiny)) == [0, 0, 0, 0x80, 0x80]
    big = np.array([1024.0, 3.0e38, -65504.0], np.float32)
    assert list(e4m3.encode(big)) == [0x7E, 0x7E, 0xFE]


def test_nearest_search_is_not_the_oracle():
    # the independent search must itself see the tie rule: a plausible
    # mistake (round half up) would flip these
    v = np.array([1.0625, 17.0, 2.0 ** -10, 3 * 2.0 ** -10], np.float32)
    assert list(nearest_code(v)) == [0x38, 0x58, 0x00, 0x02]
