"""The Python binding checks caller-supplied outputs and workspaces before
their pointers reach a kernel: wrong shape, dtype, device or layout raises,
and nothing is launched (GPU only: the inputs must be device tensors)."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
from tests.helpers import bf16_to_dev, binding, f32_to_dev, say, to_bf16_bits, u8_to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_act_quant_outputs_checked():
    fb = binding()
    say("binding: act-quant out= checks")
    x = bf16_to_dev(synth.gen_c1()["a"])                    # [32, 512]
    q = torch.empty((32, 512), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((32, 4), dtype=torch.float32, device=DEV)
    fb.fp8_act_quant_block(x, out=(q, s))                   # the right ones pass
    for bad, err in (((torch.empty((32, 256), dtype=q.dtype, device=DEV), s), ValueError),
                     ((q, torch.empty((32, 3), dtype=torch.float32, device=DEV)), ValueError),
                     ((q, torch.empty((32, 4), dtype=torch.float16, device=DEV)), TypeError),
                     ((q, torch.empty((32, 4), dtype=torch.float32)), ValueError),
                     ((torch.empty((512, 32), dtype=q.dtype, device=DEV).t(), s), ValueError)):
        with pytest.raises(err):
            fb.fp8_act_quant_block(x, out=bad)
    torch.cuda.synchronize()


def test_gemm_out_and_workspace_checked():
    fb = binding()
    say("binding: GEMM out= and workspace checks")
    # M = 48, N = 2304: the split-K decode path, which needs a workspace
    rng = np.random.default_rng(48)
    qa, sa = quant.act_quant_block(synth.f64_to_bf16_bits(rng.standard_normal((48, 1024)) * 3))
    qw, sw = quant.weight_quant_block(synth.f64_to_bf16_bits(rng.standard_normal((2304, 1024)) * 0.02))
    args = (u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    M, N = qa.shape[0], qw.shape[0]
    with pytest.raises(ValueError):
        fb.fp8_gemm_blockscaled(*args, out=torch.empty((M, N - 128), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(TypeError):
        fb.fp8_gemm_blockscaled(*args, out=torch.empty((M, N), dtype=torch.float32, device=DEV))
    with pytest.raises(ValueError):
        fb.fp8_gemm_blockscaled(*args, out=torch.empty((M, N), dtype=torch.bfloat16))
    wsb = fb.fp8_gemm_blockscaled_workspace_bytes(M, N, qa.shape[1])
    with pytest.raises(ValueError):
        fb.fp8_gemm_blockscaled(*args, workspace=torch.empty((wsb,), dtype=torch.uint8))
    # any dtype serves as workspace: its size in bytes is what counts
    ws64 = torch.empty(((wsb + 7) // 8,), dtype=torch.int64, device=DEV)
    c1 = fb.fp8_gemm_blockscaled(*args, workspace=ws64)
    c2 = fb.fp8_gemm_blockscaled(*args)
    torch.cuda.synchronize()
    assert np.array_equal(to_bf16_bits(c1), to_bf16_bits(c2))
    assert wsb > 8
    with pytest.raises(fb.Fp8bsError):      # one int64 too few
        fb.fp8_gemm_blockscaled(*args, workspace=ws64[: wsb // 8 - 1])
