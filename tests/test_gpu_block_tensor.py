"""GPU parity of fp8_act_quant_block_tensor (block and per-tensor quantization
of the same activation in one call) through the C ABI: both outputs bit for
bit against the oracle's act_quant_block and amax_quant_tensor, and against
the two separate GPU calls."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
from tests.helpers import bf16_to_dev, binding, say, to_f32, to_u8

pytestmark = pytest.mark.gpu


def run(bits, label):
    fb = binding()
    say("act_quant_block_tensor", label, bits.shape)
    qb, sb, qt, st = fb.fp8_act_quant_block_tensor(bf16_to_dev(bits))
    torch.cuda.synchronize()
    return to_u8(qb), to_f32(sb), to_u8(qt), to_f32(st)


def check_oracle(bits, label):
    qb, sb, qt, st = run(bits, label)
    qb_ref, sb_ref = quant.act_quant_block(bits)
    qt_ref, st_ref = quant.amax_quant_tensor(bits)
    assert np.array_equal(sb.view(np.uint32), sb_ref.view(np.uint32)), label
    assert np.array_equal(qb, qb_ref), label
    assert st.view(np.uint32)[0] == np.float32(st_ref).view(np.uint32), label
    assert np.array_equal(qt.reshape(-1), qt_ref.reshape(-1)), label


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (33, 2048), (128, 1024), (7, 7168)])
def test_shapes_against_oracle(M, K):
    rng = np.random.default_rng(M * 31 + K)
    check_oracle(synth.f64_to_bf16_bits(rng.standard_t(3.0, size=(M, K))), f"{M}x{K}")


def test_special_blocks_and_zero_tensor():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((40, 512))
    x[0, :128] = 0.0
    x[1, 128:256] *= 1e-30
    x[5, 300] = -6.0e4            # the tensor's amax, in one block
    x[7, :] = -0.0
    check_oracle(synth.f64_to_bf16_bits(x), "special blocks")
    check_oracle(synth.f64_to_bf16_bits(np.zeros((3, 256))), "all zero")


def test_large_m_workload_equals_separate_calls_and_oracle():
    # the large-M activation (16384 x 2048, zero and >= 1e4 blocks): equal to
    # the two separate GPU calls and to the oracle
    fb = binding()
    d = synth.gen_c5()
    x = bf16_to_dev(d["a"])
    qb, sb, qt, st = run(d["a"], "C5 A 16384x2048")
    qb2, sb2 = fb.fp8_act_quant_block(x)
    qt2, st2 = fb.fp8_amax_quant_tensor(x)
    torch.cuda.synchronize()
    assert np.array_equal(qb, to_u8(qb2)) and np.array_equal(sb.view(np.uint32), to_f32(sb2).view(np.uint32))
    assert np.array_equal(qt, to_u8(qt2)) and st.view(np.uint32)[0] == to_f32(st2).view(np.uint32)[0]
    qt_ref, st_ref = quant.amax_quant_tensor(d["a"])
    assert st.view(np.uint32)[0] == np.float32(st_ref).view(np.uint32)
    assert np.array_equal(qt, qt_ref)
    qb_ref, sb_ref = quant.act_quant_block(d["a"])
    assert np.array_equal(sb.view(np.uint32), sb_ref.view(np.uint32)) and np.array_equal(qb, qb_ref)
