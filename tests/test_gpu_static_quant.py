"""GPU parity of the per-tensor quantization with a given scale
(fp8_static_quant_tensor): bit-exact codes against the oracle through the C
ABI, for scales of every kind (the dynamic op's own, arbitrary, tiny, huge,
zero, and scales that put x/s next to e4m3 rounding midpoints), ragged sizes,
and every bf16 bit pattern; with the dynamic op's scale it reproduces the
dynamic op's bytes."""
import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, quant
from tests.helpers import bf16_to_dev, binding, f32_to_dev, say, to_u8

pytestmark = pytest.mark.gpu


def run_static(x_dev, s, label):
    fb = binding()
    say("static_quant_tensor", label, tuple(x_dev.shape), float(s))
    q = fb.fp8_static_quant_tensor(x_dev, f32_to_dev(np.array([s], np.float32)))
    torch.cuda.synchronize()
    return to_u8(q)


def check(bits, s, label):
    got = run_static(bf16_to_dev(bits), s, label)
    want = quant.static_quant_tensor(bits, np.float32(s))
    bad = np.argwhere(got != want)
    assert bad.shape[0] == 0, (label, float(s), bad.shape[0], bad[:5].tolist())


@pytest.mark.parametrize("M", [1, 64, 256, 1024, 65536])
def test_c2_sweep_reproduces_the_dynamic_op(M):
    fb = binding()
    bits = synth.gen_c2(M)["x"]
    x = bf16_to_dev(bits)
    say("amax_quant_tensor then static_quant_tensor", M)
    q_dyn, s_dyn = fb.fp8_amax_quant_tensor(x)
    q_st = fb.fp8_static_quant_tensor(x, s_dyn)        # the scale stays on the device
    torch.cuda.synchronize()
    assert np.array_equal(to_u8(q_st), to_u8(q_dyn)), M
    if M <= 1024:
        assert np.array_equal(to_u8(q_st), quant.static_quant_tensor(bits, s_dyn.cpu().numpy()[0]))


@pytest.mark.parametrize("numel", [(1 << 27) - 3, (1 << 27) + 5])
def test_both_store_forms_reproduce_the_dynamic_op(numel):
    # either side of the switch to non-temporal code stores (2^27 elements),
    # with ragged tails; the dynamic op's bytes are the reference
    fb = binding()
    g = torch.Generator(device="cuda:0").manual_seed(numel)
    x = (torch.randn(numel, generator=g, device="cuda:0") * 2.5).to(torch.bfloat16)
    say("amax_quant_tensor then static_quant_tensor", numel)
    q_dyn, s_dyn = fb.fp8_amax_quant_tensor(x)
    q_st = fb.fp8_static_quant_tensor(x, s_dyn)
    torch.cuda.synchronize()
    assert torch.equal(q_st.view(torch.uint8), q_dyn.view(torch.uint8)), numel
    tail = x[-(numel % 8 + 8):].cpu().view(torch.int16).numpy().view(np.uint16)
    want = quant.static_quant_tensor(tail, s_dyn.cpu().numpy()[0])
    assert np.array_equal(to_u8(q_st[-(numel % 8 + 8):]), want)


@pytest.mark.parametrize("numel", [1, 7, 8, 9, 511, 512, 513, 1000, 4103, 65_537, 1_000_003, 5 * (1 << 20) + 5])
def test_scales_and_ragged_sizes(numel):
    rng = np.random.default_rng(numel)
    x = rng.standard_normal(numel) * np.exp(rng.uniform(-12, 8, numel))
    bits = synth.f64_to_bf16_bits(x)
    for s in (0.0123, 1.0, 0.5, 7.3e-3, 2.0 ** -70, 3.7e4, 0.0):
        check(bits, s, f"numel={numel}")


def test_every_bf16_pattern():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = b[((b >> 7) & 0xFF) != 0xFF]                   # finite values only
    for s in (0.0123, 1e-3, 3.0e-39, 1.0, 65.5):
        check(bits, s, "all finite bf16")


def test_scales_next_to_e4m3_midpoints():
    # x / s within a few binary32 steps of a midpoint between e4m3 values:
    # the quotient's binary32 rounding decides the code
    xb = np.arange(0x3F80, 0x4000, dtype=np.uint16)
    xb = np.concatenate([xb, xb | 0x8000])
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    pos = e4m3.DECODE[:0x7F].astype(np.float64)
    mids = (pos[0x30:0x48] + pos[0x31:0x49]) / 2
    rng = np.random.default_rng(31)
    for x0 in rng.choice(xf[:128], 6, replace=False):
        for t in mids:
            s0 = np.float32(x0 / t)
            for k in (-1, 0, 1):
                s = s0 if k == 0 else np.nextafter(s0, np.float32(np.inf if k > 0 else 0), dtype=np.float32)
                check(xb, s, f"midpoint x0={x0} t={t} k={k}")


def test_caller_outputs_and_shapes():
    fb = binding()
    bits = synth.f64_to_bf16_bits(np.random.default_rng(5).standard_normal((37, 130)) * 4)
    x = bf16_to_dev(bits)
    s = f32_to_dev(np.array([0.031], np.float32))
    out = torch.full((37, 130), 0xAA, dtype=torch.uint8, device="cuda:0")
    say("static_quant_tensor with out", bits.shape)
    q = fb.fp8_static_quant_tensor(x, s, out=out)
    torch.cuda.synchronize()
    assert q is out
    assert np.array_equal(to_u8(out), quant.static_quant_tensor(bits, np.float32(0.031)))
    with pytest.raises(ValueError):
        fb.fp8_static_quant_tensor(x, f32_to_dev(np.array([1.0, 2.0], np.float32)))
    with pytest.raises(ValueError):
        fb.fp8_static_quant_tensor(x, s, out=torch.empty((37, 129), dtype=torch.uint8, device="cuda:0"))
