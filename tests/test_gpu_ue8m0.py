"""GPU parity of the power-of-two ("ue8m0") scale variants against the oracle,
through the C ABI: bit-exact codes and scales of the block and weight
quantizers, and the GEMM whose matrix cores apply the scales (M > 64) or
whose FMA path does (decode shapes) within the comparison rule, with the
accumulation term of the chained matrix-core accumulator where the matrix
cores carry it (oracle.gemm). Every output is compared."""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm, quant
from tests.helpers import (bf16_to_dev, binding, f32_to_dev, report, say, to_bf16_bits, to_f32, to_u8,
                           u8_to_dev)

pytestmark = pytest.mark.gpu


def check_block(bits, label):
    fb = binding()
    say("act_quant_block_ue8m0", label, bits.shape)
    q, s = fb.fp8_act_quant_block_ue8m0(bf16_to_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.act_quant_block_ue8m0(bits)
    gs = to_f32(s)
    bad_s = np.nonzero(gs.view(np.uint32) != s_ref.view(np.uint32))
    assert bad_s[0].size == 0, (label, "scales differ", bad_s[0][:5], bad_s[1][:5], gs[bad_s][:3], s_ref[bad_s][:3])
    bad = np.argwhere(to_u8(q) != q_ref)
    assert bad.shape[0] == 0, (label, "codes differ", bad[:5].tolist())


def test_block_quant_workloads():
    check_block(synth.gen_c1()["a"], "C1")
    check_block(synth.gen_c3(64)["a"], "C3 M=64")
    check_block(synth.gen_c4()["a"], "C4")
    check_block(synth.gen_c5()["a"], "C5")


def test_block_quant_edges():
    rng = np.random.default_rng(21)
    rows = []
    for k in (-130, -127, -126, -100, -8, 0, 8, 100, 119):
        for f in (1.0, 1.0 + 2.0 ** -7, 1.0 - 2.0 ** -8):           # amax/448 at, above, below 2^k
            r = rng.uniform(-1, 1, 128) * 448.0 * 2.0 ** k * f
            r[rng.integers(0, 128)] = 448.0 * 2.0 ** k * f * rng.choice([-1, 1])
            rows.append(r)
    rows.append(np.zeros(128))
    rows.append(np.full(128, -0.0))
    rows.append(np.ldexp(rng.uniform(-1, 1, 128), -133))            # bf16 subnormals
    rows.append(rng.standard_normal(128) * 3e38 / 4)                 # near the bf16 maximum
    bits = synth.f64_to_bf16_bits(np.array(rows))
    check_block(bits, "edge blocks")
    check_block(np.concatenate([synth.special_blocks()] * 1, axis=0), "special blocks")


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (1000, 128), (7, 7168)])
def test_block_quant_ragged(M, K):
    rng = np.random.default_rng(M * K)
    check_block(synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * np.exp(rng.uniform(-30, 30, (M, 1)))),
                f"{M}x{K}")


def test_weight_quant():
    fb = binding()
    rng = np.random.default_rng(22)
    w = rng.standard_normal((256, 384)) * 0.02
    w[:128, :128] = 0.0
    w[128:, 128:256] *= 1e-30
    w[:128, 256:] *= 1e4
    for label, bits in (("C3 W", synth.gen_c3(1)["w"]), ("special", synth.f64_to_bf16_bits(w))):
        say("weight_quant_block_ue8m0", label, bits.shape)
        q, s = fb.fp8_weight_quant_block_ue8m0(bf16_to_dev(bits))
        torch.cuda.synchronize()
        q_ref, s_ref = quant.weight_quant_block_ue8m0(bits)
        assert np.array_equal(to_f32(s).view(np.uint32), s_ref.view(np.uint32)), label
        assert np.array_equal(to_u8(q), q_ref), label


def operands(a_bits, w_bits, w_scale_exp=None):
    qa, sa = quant.act_quant_block_ue8m0(a_bits)
    qw, sw = quant.weight_quant_block_ue8m0(w_bits)
    if w_scale_exp is not None:
        sw = np.ldexp(np.float32(1.0), w_scale_exp).astype(np.float32)
    return qa, sa, qw, sw


def run(qa, sa, qw, sw, label):
    fb = binding()
    say("gemm_blockscaled_ue8m0", label, qa.shape, qw.shape)
    c = fb.fp8_gemm_blockscaled_ue8m0(u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    torch.cuda.synchronize()
    return to_bf16_bits(c)


def check(qa, sa, qw, sw, label):
    c = run(qa, sa, qw, sw, label)
    # the matrix cores carry the accumulator over the K blocks where the
    # tiled kernel runs (M > 64); decode shapes run the FMA kernels
    res = gemm.compare_gemm_full(c, qa, sa, qw, sw, chained=qa.shape[0] > 64)
    report(label, res)
    assert res["ok"], (label, res)


@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (32, 512, 512), (64, 256, 2048), (12, 256, 128 * 9),
                                   (24, 384, 2048), (48, 2048, 7168), (40, 2304, 1280), (128, 2048, 2048),
                                   (300, 384, 2048),
                                   (96, 256, 512), (300, 384, 1024), (520, 640, 4096),
                                   (300, 384, 2432)])
def test_gemm_shapes(M, N, K):
    rng = np.random.default_rng(M + 3 * N + K)
    a = synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 3)
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    check(*operands(a, w), f"{M}x{N}x{K}")


def test_gemm_prefill():
    d = synth.gen_c4()
    check(*operands(d["a"], d["w"]), "C4 shape")


def test_gemm_large_tiles_ragged_k_blocks():
    # 256 x 256 tiles, ragged M, 13 K blocks (activation-scale chunks of 8)
    M, N, K = 4133, 4096, 1664
    rng = np.random.default_rng(1664)
    a = synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 3)
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    check(*operands(a, w), f"{M}x{N}x{K}")


def test_gemm_large_m_drawn_scales():
    # the large-M workload's structure with power-of-two weight scales drawn
    # log-uniform over the same range (2^-14 .. 2^-3)
    d = synth.gen_c5()
    rng = np.random.default_rng(5)
    exps = rng.integers(-14, -3, (7168 // 128, 2048 // 128))
    check(*operands(d["a"], d["w"], w_scale_exp=exps), "C5 shape")


def test_gemm_zero_and_tiny_scales():
    rng = np.random.default_rng(23)
    a = rng.standard_normal((128, 512))
    a[:, :128] = 0.0                                   # zero blocks (scale 0)
    a[:64, 128:256] *= 1e-35                           # scales near 2^-127
    qa, sa, qw, sw = operands(synth.f64_to_bf16_bits(a), synth.f64_to_bf16_bits(rng.standard_normal((256, 512)) * 0.02))
    check(qa, sa, qw, sw, "zero and tiny scales")
