"""The allocation-free per-tensor quantization (fp8_amax_quant_tensor_noalloc,
its first pass's partial maxima in the library's own device array) through
the C ABI: bit for bit the output of fp8_amax_quant_tensor (caller's
workspace), on consecutive calls whose inputs shrink, so that a later call
would show any use of the partial maxima an earlier call left behind."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import quant
from tests.helpers import bf16_to_dev, binding, say, to_u8

pytestmark = pytest.mark.gpu


def noalloc_c(L, x):
    """The raw C call, outputs allocated here (the call itself allocates nothing)."""
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty((1,), dtype=torch.float32, device=x.device)
    rc = L.fp8_amax_quant_tensor_noalloc(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(s.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.fp8bs_status_string(rc).decode()
    return q, s


def test_noalloc_equals_workspace_entry_point():
    fb = binding()
    L = fb.lib()
    rng = np.random.default_rng(99)
    # shrinking inputs; the earlier ones have the larger maxima, so stale
    # partial maxima would raise a later call's scale
    cases = [("per-tensor sweep M=65536", synth.gen_c2(65536)["x"], 1000.0),
             ("M=1024", synth.gen_c2(1024)["x"], 10.0),
             ("ragged 300001 elements", synth.f64_to_bf16_bits(rng.standard_normal(300001)), 1.0),
             ("one launch, several workgroups, 40009 elements", synth.f64_to_bf16_bits(rng.standard_normal(40009)), 1.0),
             ("small path 4099 elements", synth.f64_to_bf16_bits(rng.standard_normal(4099)), 1.0)]
    for label, bits, mul in cases:
        x = bf16_to_dev(bits) * mul
        say("amax_quant_tensor_noalloc", label, tuple(x.shape))
        q1, s1 = noalloc_c(L, x)
        q2, s2 = fb.fp8_amax_quant_tensor(x)
        torch.cuda.synchronize()
        assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), label
        assert torch.equal(q1, q2.view(torch.uint8)), label
    # the last two calls against the oracle as well
    for label, bits in (("M=1024", synth.gen_c2(1024)["x"]),
                        ("ragged", synth.f64_to_bf16_bits(rng.standard_normal(70001)))):
        x = bf16_to_dev(bits)
        q1, s1 = noalloc_c(L, x)
        torch.cuda.synchronize()
        q_ref, s_ref = quant.amax_quant_tensor(bits)
        assert np.array_equal(to_u8(q1).reshape(q_ref.shape), q_ref), label
        assert s1.cpu().numpy()[0] == s_ref, label


def test_binding_noalloc_with_outputs_given():
    fb = binding()
    x = bf16_to_dev(synth.gen_c2(256)["x"])
    q = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device="cuda:0")
    s = torch.empty((1,), dtype=torch.float32, device="cuda:0")
    fb.fp8_amax_quant_tensor_noalloc(x, out=(q, s))
    q2, s2 = fb.fp8_amax_quant_tensor(x)
    torch.cuda.synchronize()
    assert torch.equal(q.view(torch.uint8), q2.view(torch.uint8)) and torch.equal(s, s2)
