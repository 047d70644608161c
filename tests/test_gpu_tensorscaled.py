"""GPU parity of the per-tensor-scaled FP8 GEMM (the consumer of the per-tensor
quantization) against the oracle, through the C ABI. Operands quantized by the
oracle; one case chains the GPU per-tensor quantizer into the GEMM."""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm, quant
from tests.helpers import (bf16_to_dev, binding, f32_to_dev, say, to_bf16_bits, u8_to_dev)

pytestmark = pytest.mark.gpu


def check(qa, sa, qw, sw, label, rows=None):
    fb = binding()
    say("gemm_tensorscaled", label, qa.shape, qw.shape)
    c = fb.fp8_gemm_tensorscaled(u8_to_dev(qa), f32_to_dev(np.array([sa], np.float32)), u8_to_dev(qw),
                                 f32_to_dev(np.array([sw], np.float32)))
    torch.cuda.synchronize()
    c = to_bf16_bits(c)
    if rows is not None:
        c, qa = c[rows], qa[rows]
    R = gemm.gemm_tensorscaled_ref(qa, sa, qw, sw)
    S = gemm.gemm_tensorscaled_abs_ref(qa, sa, qw, sw)
    Se = gemm.gemm_exp_envelope_ref(qa, np.full((qa.shape[0], qa.shape[1] // 128), sa, np.float32), qw,
                                    np.full((qw.shape[0] // 128, qw.shape[1] // 128), sw, np.float32))
    res = gemm.compare_gemm(c, R, S, qa.shape[1], Se, chained=True)
    say("  ", label, {k: res[k] for k in res if k != "ok"})
    assert res["ok"], (label, res)


def tensor_operands(a_bits, w_bits):
    qa, sa = quant.amax_quant_tensor(a_bits)
    qw, sw = quant.amax_quant_tensor(w_bits)
    return qa, sa, qw, sw


@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (16, 512, 1024), (4, 128, 128 * 400), (64, 2048, 2048), (33, 256, 640),
                                   (96, 256, 512), (300, 384, 1024), (1000, 1024, 2048)])
def test_shapes(M, N, K):
    rng = np.random.default_rng(M * 5 + N + K)
    a = synth.f64_to_bf16_bits(rng.standard_normal((M, K)))
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    check(*tensor_operands(a, w), f"{M}x{N}x{K}")


def test_decode_activation_from_gpu_quantizer():
    # the pages' decode shape [64, 2048]: the GPU per-tensor quantizer feeds the GEMM
    fb = binding()
    a = synth.gen_c2(64)["x"]
    w = synth.f64_to_bf16_bits(np.random.default_rng(7).standard_normal((2048, 2048)) * 0.02)
    q, s = fb.fp8_amax_quant_tensor(bf16_to_dev(a))
    qw, sw = quant.amax_quant_tensor(w)
    c = fb.fp8_gemm_tensorscaled(q, s, u8_to_dev(qw), f32_to_dev(np.array([sw], np.float32)))
    torch.cuda.synchronize()
    qa, sa = quant.amax_quant_tensor(a)
    R = gemm.gemm_tensorscaled_ref(qa, sa, qw, sw)
    S = gemm.gemm_tensorscaled_abs_ref(qa, sa, qw, sw)
    Se = gemm.gemm_exp_envelope_ref(qa, np.full((64, 16), sa, np.float32), qw, np.full((16, 16), sw, np.float32))
    res = gemm.compare_gemm(to_bf16_bits(c), R, S, 2048, Se, chained=True)
    assert res["ok"], res


def test_large_sampled_rows():
    d = synth.gen_c5()
    rows = np.random.default_rng(8).choice(16384, 24, replace=False)
    check(*tensor_operands(d["a"], d["w"]), "C5 shape, per-tensor scales", rows=rows)
