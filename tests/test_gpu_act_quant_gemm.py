"""GPU parity of the fused block act-quant + GEMM entry point
(fp8_act_quant_gemm_blockscaled) through the C ABI.

The oracle quantizes x with the 1x128 block rule and multiplies in fp64; the
comparison rule is the GEMM's (oracle.gemm.compare_gemm). Where the call runs
as one kernel (M <= 8, x's codes in LDS) its output must also equal, bit for
bit, the two-call path on the GPU (fp8_act_quant_block, then
fp8_gemm_blockscaled), which performs the same operations in the same order.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm, quant
from tests.helpers import bf16_to_dev, binding, report, say, to_bf16_bits

pytestmark = pytest.mark.gpu


def weights(rng, N, K):
    qw, sw = quant.weight_quant_block(synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02))
    return qw, sw


def run_fused(x_bits, qw, sw, label, workspace=None):
    fb = binding()
    say("act_quant_gemm_blockscaled", label, x_bits.shape, qw.shape)
    c = fb.fp8_act_quant_gemm_blockscaled(bf16_to_dev(x_bits), torch.from_numpy(qw).to("cuda:0"),
                                          torch.from_numpy(sw).to("cuda:0"), workspace=workspace)
    torch.cuda.synchronize()
    return to_bf16_bits(c)


def run_two_calls(x_bits, qw, sw):
    fb = binding()
    qa, sa = fb.fp8_act_quant_block(bf16_to_dev(x_bits))
    c = fb.fp8_gemm_blockscaled(qa, sa, torch.from_numpy(qw).to("cuda:0"), torch.from_numpy(sw).to("cuda:0"))
    torch.cuda.synchronize()
    return to_bf16_bits(c)


def check_oracle(c, x_bits, qw, sw, label):
    qa, sa = quant.act_quant_block(x_bits)
    res = gemm.compare_gemm_full(c, qa, sa, qw, sw)
    report(label, res)
    assert res["ok"], (label, res)


@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 9, 16])
def test_decode_workload(M):
    # the decode workload's shapes and distributions (N=2048, K=7168); one
    # kernel up to M = 8, two launches from M = 9
    d = synth.gen_c3(M)
    qw, sw = quant.weight_quant_block(d["w"])
    c = run_fused(d["a"], qw, sw, f"C3 M={M}")
    check_oracle(c, d["a"], qw, sw, f"C3 M={M}")
    assert np.array_equal(c, run_two_calls(d["a"], qw, sw)), "one-kernel path differs from the two calls"


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 384), (4, 384, 35712), (3, 640, 128 * 7),
                                   (4, 128, 35840), (7, 640, 2560), (8, 384, 17792), (8, 128, 17920),
                                   (5, 256, 128 * 200), (2, 256, 128 * 301), (9, 256, 1024), (40, 384, 2048),
                                   (64, 2048, 7168),
                                   (300, 512, 1024)])
def test_shapes(M, N, K):
    # (4, 384, 35712) and (8, 384, 17792): largest K that runs as one kernel
    # at M = 4 and 8; K = 7 blocks leaves the last pair of packed K blocks
    # half empty; K = 200 and 301 blocks take four steps in flight per wave;
    # (4, 128, 35840), (8, 128, 17920) and M > 8: act-quant and GEMM through
    # the workspace
    rng = np.random.default_rng(M * 7 + N + K)
    x = synth.f64_to_bf16_bits(rng.standard_t(3.0, size=(M, K)))
    qw, sw = weights(rng, N, K)
    c = run_fused(x, qw, sw, f"{M}x{N}x{K}")
    check_oracle(c, x, qw, sw, f"{M}x{N}x{K}")
    assert np.array_equal(c, run_two_calls(x, qw, sw))


def test_special_blocks():
    # all-zero blocks (scale 0), blocks with a maximum near 1e-30 (scale
    # below 2^-64: the IEEE quotient), a block with one huge element, and a
    # negative-zero-only block. (Scales whose product with the weight scale
    # falls below fp32's normal range are left out: the fp32 scale product
    # then keeps only a few significant bits, which no bf16 bound covers.)
    rng = np.random.default_rng(99)
    M, N, K = 6, 256, 1024
    x = rng.standard_normal((M, K))
    x[0, :128] = 0.0
    x[1, 128:256] *= 1e-30
    x[2, 256:384] = 0.0
    x[2, 300] = 3.0e4
    x[3, 384:512] = -0.0
    x[4] *= 1e-25
    xb = synth.f64_to_bf16_bits(x)
    qw, sw = weights(rng, N, K)
    c = run_fused(xb, qw, sw, "special blocks")
    check_oracle(c, xb, qw, sw, "special blocks")
    assert np.array_equal(c, run_two_calls(xb, qw, sw))


def test_workspace_reuse_across_sizes():
    # one caller-owned workspace, two calls through it (the larger first)
    fb = binding()
    rng = np.random.default_rng(5)
    big = (48, 512, 2048)
    small = (20, 256, 1024)
    ws = torch.empty((fb.fp8_act_quant_gemm_blockscaled_workspace_bytes(*big),), dtype=torch.uint8,
                     device="cuda:0")
    assert fb.fp8_act_quant_gemm_blockscaled_workspace_bytes(*small) <= ws.numel()
    for M, N, K in (big, small):
        x = synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 4)
        qw, sw = weights(rng, N, K)
        c = run_fused(x, qw, sw, f"reuse {M}x{N}x{K}", workspace=ws)
        check_oracle(c, x, qw, sw, f"reuse {M}x{N}x{K}")
