"""GPU parity of the quantizers against the CPU oracle: bit-exact e4m3 bytes
and fp32 scales, through the C ABI (binding -> libfp8bs.so)."""
import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, quant
from tests.helpers import (bf16_to_dev, binding, f32_to_dev, say, to_f32, to_u8)

pytestmark = pytest.mark.gpu


def check_block(bits, label):
    fb = binding()
    say("act_quant_block", label, bits.shape)
    q, s = fb.fp8_act_quant_block(bf16_to_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.act_quant_block(bits)
    gq, gs = to_u8(q), to_f32(s)
    assert gs.shape == s_ref.shape
    bad_s = np.nonzero(gs.view(np.uint32) != s_ref.view(np.uint32))
    assert bad_s[0].size == 0, (label, "scales differ", bad_s[0][:5], bad_s[1][:5])
    bad = np.argwhere(gq != q_ref)
    assert bad.shape[0] == 0, (label, "codes differ", bad[:5].tolist(),
                               gq[tuple(bad[0])] if len(bad) else None,
                               q_ref[tuple(bad[0])] if len(bad) else None)


def test_block_quant_c1():
    check_block(synth.gen_c1()["a"], "C1 32x512")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_block_quant_c3(M):
    check_block(synth.gen_c3(M)["a"], f"C3 M={M}")


def test_block_quant_c4_full():
    check_block(synth.gen_c4()["a"], "C4 4096x7168")


def test_block_quant_c5_full():
    check_block(synth.gen_c5()["a"], "C5 16384x2048")


def test_block_quant_quotient_grid():
    # every (significand of block max, significand of element) pair, both
    # signs, 15 binades, block maxima from 2**-126 to 2**100 (both the fast
    # quotient and the IEEE-division path for tiny scales)
    g = synth.quotient_grid()
    n10 = (g.shape[0] // 10) * 10
    check_block(g[:n10].reshape(-1, 1280), "quotient grid, 10 blocks per row")
    check_block(g, "quotient grid rows")


def test_block_quant_special_blocks():
    sb = synth.special_blocks()
    check_block(sb, "special blocks")
    check_block(np.tile(sb, (3, 4)), "special blocks tiled")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (33, 256), (1000, 128), (7, 7168)])
def test_block_quant_ragged(M, K):
    rng = np.random.default_rng(M * 1000 + K)
    x = rng.standard_t(3.0, size=(M, K)) * 10.0 ** rng.uniform(-3, 3, size=(M, 1))
    check_block(synth.f64_to_bf16_bits(x), f"ragged {M}x{K}")


def test_block_quant_deterministic():
    fb = binding()
    x = bf16_to_dev(synth.gen_c3(64)["a"])
    q1, s1 = fb.fp8_act_quant_block(x)
    q2, s2 = fb.fp8_act_quant_block(x)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s1, s2)


def test_weight_quant_parity():
    fb = binding()
    for label, w in (("C1 W", synth.gen_c1()["w"]), ("C3 W", synth.gen_c3(1)["w"]),
                     ("C5 W", synth.gen_c5(M=128)["w"])):
        say("weight_quant_block", label, w.shape)
        q, s = fb.fp8_weight_quant_block(bf16_to_dev(w))
        torch.cuda.synchronize()
        q_ref, s_ref = quant.weight_quant_block(w)
        assert np.array_equal(to_f32(s).view(np.uint32), s_ref.view(np.uint32)), label
        assert np.array_equal(to_u8(q), q_ref), label


def test_weight_quant_special():
    fb = binding()
    rng = np.random.default_rng(4)
    w = rng.standard_normal((256, 384)) * 0.02
    w[:128, :128] = 0.0                                 # all-zero block
    w[128:, 128:256] *= 1e-30                           # tiny block: IEEE-division path
    w[:128, 256:] *= 1e4
    bits = synth.f64_to_bf16_bits(w)
    q, s = fb.fp8_weight_quant_block(bf16_to_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.weight_quant_block(bits)
    assert np.array_equal(to_f32(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(to_u8(q), q_ref)


def test_encode_exhaustive_rounding_range():
    """The library's fp32 -> e4m3 step against the oracle encoder on every
    positive float32 in [2**-12, 2**10), their negatives, and random bit
    patterns over the whole finite range."""
    fb = binding()
    lo, hi = (127 - 12) << 23, (127 + 10) << 23
    step = 1 << 24
    for start in range(lo, hi, step):
        bits = np.arange(start, min(start + step, hi), dtype=np.uint32)
        v = bits.view(np.float32)
        for sign in (1.0, -1.0):
            vv = (v * np.float32(sign)).astype(np.float32)
            got = to_u8(fb.debug_encode_e4m3(f32_to_dev(vv)))
            want = e4m3.encode(vv)
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (hex(start), sign, vv[bad[:4]], got[bad[:4]], want[bad[:4]])
    rng = np.random.default_rng(17)
    b = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    v = b.view(np.float32)
    v = v[np.isfinite(v)]
    v = v[: len(v) - (len(v) % 4) - 1]                  # length 3 mod 4: a ragged tail
    got = to_u8(fb.debug_encode_e4m3(f32_to_dev(v)))
    assert np.array_equal(got, e4m3.encode(v))


def test_signed_zeros_in_nonzero_blocks():
    # -0 and +0 inside ordinary blocks (the three-operation quotient path)
    rng = np.random.default_rng(21)
    bits = synth.f64_to_bf16_bits(rng.standard_normal((64, 1024)))
    bits[:, ::5] = 0x8000
    bits[:, 1::7] = 0x0000
    check_block(bits, "signed zeros")
    fb = binding()
    say("amax_quant_tensor", "signed zeros")
    q, s = fb.fp8_amax_quant_tensor(bf16_to_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.amax_quant_tensor(bits)
    assert np.array_equal(to_u8(q), q_ref) and to_f32(s)[0] == s_ref


def check_block_f32(x, label):
    fb = binding()
    say("act_quant_block_f32", label, x.shape)
    q, s = fb.fp8_act_quant_block_f32(torch.from_numpy(np.ascontiguousarray(x, np.float32)).to("cuda:0"))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.act_quant_block_f32(x)
    assert np.array_equal(to_f32(s).view(np.uint32), s_ref.view(np.uint32)), label
    bad = np.argwhere(to_u8(q) != q_ref)
    assert bad.shape[0] == 0, (label, bad[:5].tolist())


def test_block_quant_f32_input():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((257, 1024)) * np.exp(rng.uniform(-40, 40, (257, 1)))).astype(np.float32)
    x[5, 128:256] = 0.0                                  # zero block
    x[6, :128] = -0.0
    x[7, 256:384] *= np.float32(1e-30)                   # small scales
    x[8, :128] = np.float32(448.0) * (1 + rng.integers(0, 2, 128) * 2.0 ** -20)   # near-ties
    check_block_f32(x, "f32 mixed")
    check_block_f32(rng.standard_normal((1024, 128)).astype(np.float32), "f32 [1024, 128] (the page's example shape)")
