"""GPU parity of the per-tensor quantizer (exact amax over the whole tensor):
bit-exact bytes and scale against the oracle, through the C ABI; the amax
stage alone (fp8_amax_tensor) gives the exact maximum and the same scale."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
from tests.helpers import bf16_to_dev, binding, say, to_f32, to_u8

pytestmark = pytest.mark.gpu


def check_tensor(bits, label):
    fb = binding()
    say("amax_quant_tensor", label, bits.shape)
    q, s = fb.fp8_amax_quant_tensor(bf16_to_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = quant.amax_quant_tensor(bits)
    gs = to_f32(s)
    assert gs.shape == (1,)
    assert gs.view(np.uint32)[0] == np.float32(s_ref).view(np.uint32), (label, gs[0], s_ref)
    gq = to_u8(q)
    bad = np.argwhere(gq != q_ref)
    assert bad.shape[0] == 0, (label, bad[:5].tolist())
    # the amax stage alone (fp8_amax_tensor): the exact maximum and the same scale
    amax, s2 = fb.fp8_amax_tensor(bf16_to_dev(bits))
    torch.cuda.synchronize()
    want = np.float32(np.max(np.abs(synth.bf16_bits_to_f64(bits))))
    assert to_f32(amax).view(np.uint32)[0] == want.view(np.uint32), (label, to_f32(amax)[0], want)
    assert to_f32(s2).view(np.uint32)[0] == np.float32(s_ref).view(np.uint32), label


@pytest.mark.parametrize("M", [1, 64, 256, 1024, 65536])
def test_c2_sweep(M):
    check_tensor(synth.gen_c2(M)["x"], f"C2 M={M}")


def test_c5_activation():
    check_tensor(synth.gen_c5()["a"], "C5 A 16384x2048")


# the three forms: one workgroup (up to 2^14 elements), several workgroups that
# each read the whole tensor (up to 2^16), two passes (above); sizes on both
# sides of each switch, ragged tails, shares of the mid form that end early
@pytest.mark.parametrize("numel", [1, 7, 8, 9, 127, 1000, (1 << 14) - 1, 1 << 14, (1 << 14) + 1,
                                   (1 << 14) + 8, 20_007, 40_000, (1 << 16) - 3, 1 << 16, (1 << 16) + 1,
                                   (1 << 16) + 8, (1 << 17) - 1, 1 << 17,
                                   (1 << 17) + 1, (1 << 17) + 7, 1_000_003, 5 * (1 << 20) + 5])
def test_ragged_numel(numel):
    rng = np.random.default_rng(numel)
    x = rng.standard_normal(numel) * 3.0
    x[rng.integers(0, numel)] = -1234.5             # the maximum, anywhere
    check_tensor(synth.f64_to_bf16_bits(x), f"numel={numel}")


def test_max_in_the_tail():
    numel = (1 << 20) + 5
    x = np.random.default_rng(1).standard_normal(numel)
    x[-1] = 9e3                                       # beyond the last 16-byte vector
    check_tensor(synth.f64_to_bf16_bits(x), "max in tail")


@pytest.mark.parametrize("numel", [100, 50_001, (1 << 17) + 9, 3 << 20])
def test_all_zero_and_tiny(numel):
    check_tensor(np.zeros(numel, np.uint16), f"zeros {numel}")
    neg0 = np.full(numel, 0x8000, np.uint16)
    check_tensor(neg0, f"neg zeros {numel}")
    rng = np.random.default_rng(2)
    tiny = synth.f64_to_bf16_bits(rng.standard_normal(numel) * 1e-30)   # IEEE path
    check_tensor(tiny, f"tiny {numel}")


def test_deterministic_and_reusable_workspace():
    # one workspace, garbage on entry, reused across calls of different sizes
    fb = binding()
    sizes = (1 << 20, (3 << 20) + 9, 40_000, 1 << 22)
    wsb = max(fb.fp8_amax_quant_tensor_workspace_bytes(n) for n in sizes)
    ws = torch.full((wsb,), 255, dtype=torch.uint8, device="cuda:0")
    x = bf16_to_dev(synth.gen_c2(1024)["x"])
    q1, s1 = fb.fp8_amax_quant_tensor(x, workspace=ws)
    q2, s2 = fb.fp8_amax_quant_tensor(x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(q1.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s1, s2)
    rng = np.random.default_rng(5)
    for n in sizes:
        bits = synth.f64_to_bf16_bits(rng.standard_normal(n) * 2.0)
        q, s = fb.fp8_amax_quant_tensor(bf16_to_dev(bits), workspace=ws)
        torch.cuda.synchronize()
        q_ref, s_ref = quant.amax_quant_tensor(bits)
        assert to_f32(s).view(np.uint32)[0] == np.float32(s_ref).view(np.uint32), n
        assert np.array_equal(to_u8(q), q_ref), n
