"""The C-ABI library on the host: it loads, exports every entry point that
include/fp8bs.h declares, and rejects bad arguments before touching a device
(no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest
import torch

import fp8_block_scaled_act_amd as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")

OK, ENULL, ESHAPE, EALIGN, EWS, EDEV = 0, 1, 2, 3, 4, 5
P = 0x100000          # a fake, 16-byte aligned pointer value (never dereferenced)
PU = 0x100001         # a misaligned one


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return fb.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert "fp8_act_quant_block" in names and "fp8_gemm_blockscaled" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(fb.EXPORTED_SYMBOLS)


def test_status_strings(L):
    for code in range(8):
        s = L.fp8bs_status_string(code).decode()
        assert s.startswith("FP8BS_")
    assert L.fp8bs_status_string(99).decode() == "FP8BS_ERR_UNKNOWN"


def test_act_quant_argument_errors(L):
    f = L.fp8_act_quant_block
    assert f(None, 4, 128, P, P, None) == ENULL
    assert f(P, 4, 128, None, P, None) == ENULL
    assert f(P, 4, 128, P, None, None) == ENULL
    assert f(P, 0, 128, P, P, None) == ESHAPE
    assert f(P, 4, 100, P, P, None) == ESHAPE
    assert f(P, 4, 0, P, P, None) == ESHAPE
    assert f(P, -1, 128, P, P, None) == ESHAPE
    assert f(PU, 4, 128, P, P, None) == EALIGN
    assert f(P, 4, 128, PU, P, None) == EALIGN
    assert f(P, 4, 128, P, P + 2, None) == EALIGN


def test_tensor_quant_argument_errors(L):
    f = L.fp8_amax_quant_tensor
    ws = L.fp8_amax_quant_tensor_workspace_bytes
    assert ws(1) == 0 and ws(1 << 14) == 0 and ws((1 << 14) + 1) == 0 and ws(1 << 16) == 0
    assert ws((1 << 16) + 1) == 4096
    big = 1 << 20
    assert ws(big) > 0
    assert f(None, 10, P, P, None, 0, None) == ENULL
    assert f(P, 0, P, P, None, 0, None) == ESHAPE
    assert f(PU, 10, P, P, None, 0, None) == EALIGN
    assert f(P, big, P, P, None, 0, None) == EWS
    assert f(P, big, P, P, P, ws(big) - 1, None) == EWS
    assert f(P, big, P, P, PU, ws(big), None) == EALIGN


def test_amax_only_argument_errors(L):
    f = L.fp8_amax_tensor
    big = 1 << 20
    ws = L.fp8_amax_quant_tensor_workspace_bytes(big)
    assert f(None, 10, P, P, None, 0, None) == ENULL
    assert f(P, 10, None, P, None, 0, None) == ENULL
    assert f(P, 0, P, P, None, 0, None) == ESHAPE
    assert f(PU, 10, P, P, None, 0, None) == EALIGN
    assert f(P, big, P, P, None, 0, None) == EWS
    assert f(P, big, P, P, P, ws - 1, None) == EWS
    assert f(P, big, P, P, PU, ws, None) == EALIGN


def test_tensor_quant_noalloc_argument_errors(L):
    f = L.fp8_amax_quant_tensor_noalloc
    assert f(None, 10, P, P, None) == ENULL
    assert f(P, 10, None, P, None) == ENULL
    assert f(P, 0, P, P, None) == ESHAPE
    assert f(PU, 10, P, P, None) == EALIGN
    assert f(P, 10, P, P + 2, None) == EALIGN


def test_static_quant_argument_errors(L):
    f = L.fp8_static_quant_tensor
    assert f(None, 10, P, P, None) == ENULL
    assert f(P, 10, None, P, None) == ENULL
    assert f(P, 10, P, None, None) == ENULL
    assert f(P, 0, P, P, None) == ESHAPE
    assert f(P, -3, P, P, None) == ESHAPE
    assert f(P, 1 << 42, P, P, None) == ESHAPE
    assert f(PU, 10, P, P, None) == EALIGN
    assert f(P, 10, P + 2, P, None) == EALIGN
    assert f(P, 10, P, P + 8, None) == EALIGN
    assert f(P, 10, P, P, None) == EDEV          # valid: the device check comes next


def test_gemm_argument_errors(L):
    f = L.fp8_gemm_blockscaled
    assert f(None, P, P, P, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, P, None, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, P, P, P, 0, 128, 128, None, 0, None) == ESHAPE
    assert f(P, P, P, P, P, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(P, P, P, P, P, 4, 128, 64, None, 0, None) == ESHAPE
    assert f(P, P, P, P, P, 4, 128, 130, None, 0, None) == ESHAPE
    # K above 2^22 (tile-relative copy offsets are 32-bit), tiled path (M > 64)
    assert f(P, P, P, P, P, 256, 128, (1 << 22) + 128, None, 0, None) == ESHAPE
    assert f(PU, P, P, P, P, 4, 128, 128, None, 0, None) == EALIGN
    assert f(P, P, P, P, PU, 4, 128, 128, None, 0, None) == EALIGN
    assert f(P, P + 1, P, P, P, 4, 128, 128, None, 0, None) == EALIGN


def test_weight_quant_argument_errors(L):
    f = L.fp8_weight_quant_block
    assert f(None, 128, 128, P, P, None) == ENULL
    assert f(P, 64, 128, P, P, None) == ESHAPE
    assert f(P, 128, 192, P, P, None) == ESHAPE
    assert f(PU, 128, 128, P, P, None) == EALIGN


def test_debug_mfma_block_argument_errors(L):
    f = L.fp8bs_debug_mfma_block
    assert f(None, P, P, 1, None) == ENULL
    assert f(P, P, None, 1, None) == ENULL
    assert f(P, P, P, 0, None) == ESHAPE
    assert f(P, P, P, 1 << 31, None) == ESHAPE
    assert f(PU, P, P, 1, None) == EALIGN
    assert f(P, P, P + 2, 1, None) == EALIGN


def test_debug_encode_argument_errors(L):
    f = L.fp8bs_debug_encode_e4m3
    assert f(None, P, 4, None) == ENULL
    assert f(P, P, 0, None) == ESHAPE
    assert f(PU, P, 4, None) == EALIGN


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path only")
def test_valid_arguments_without_a_device_report_device_error(L):
    # all arguments valid: the next step is the device check, which fails here
    assert L.fp8_act_quant_block(P, 4, 128, P, P, None) == EDEV
    assert L.fp8_amax_quant_tensor_noalloc(P, 1 << 20, P, P, None) == EDEV
    assert L.fp8_gemm_blockscaled(P, P, P, P, P, 4, 128, 128, None, 0, None) == EDEV


def test_python_binding_rejects_bad_tensors():
    x = torch.zeros((4, 128), dtype=torch.bfloat16)       # CPU tensor
    with pytest.raises(ValueError):
        fb.fp8_act_quant_block(x)
    with pytest.raises(TypeError):
        fb.fp8_act_quant_block(torch.zeros((4, 128), dtype=torch.float32))


def test_gemm_k_limits(L):
    # copy offsets within a tile are 32-bit: K above 2^22 is rejected
    assert L.fp8_gemm_blockscaled(P, P, P, P, P, 8, 128, (1 << 22) + 128, None, 0, None) == ESHAPE
    # 32 < M <= 64 with N > 2048 splits K into at most 32 parts of at most 16
    # blocks; M <= 32, and M <= 64 with N <= 2048, take all of K in one
    # workgroup and have no such limit
    assert L.fp8_gemm_blockscaled(P, P, P, P, P, 33, 2176, 128 * 513, None, 0, None) == ESHAPE
    assert L.fp8_gemm_blockscaled_workspace_bytes(32, 128, 128 * 513) == 0
    assert L.fp8_gemm_blockscaled_workspace_bytes(64, 2048, 128 * 513) == 0
    for M in (1, 8, 9, 16, 17, 32, 33, 48, 64):
        assert L.fp8_gemm_blockscaled_workspace_bytes(M, 2048, 7168) == 0
    assert L.fp8_gemm_blockscaled_workspace_bytes(33, 2176, 7168) > 0
    assert L.fp8_gemm_blockscaled_workspace_bytes(64, 4096, 7168) > 0
    # a shape the call rejects needs no workspace, and the act-quant + GEMM
    # call rejects it before enqueuing anything
    assert L.fp8_gemm_blockscaled_workspace_bytes(40, 2176, 128 * 513) == 0
    assert L.fp8_act_quant_gemm_blockscaled_workspace_bytes(40, 2176, 128 * 513) == 0
    assert L.fp8_act_quant_gemm_blockscaled(P, P, P, P, 40, 2176, 128 * 513, P, 1 << 30, None) == ESHAPE


def test_ue8m0_argument_errors(L):
    assert L.fp8_act_quant_block_ue8m0(None, 4, 128, P, P, None) == ENULL
    assert L.fp8_act_quant_block_ue8m0(P, 4, 100, P, P, None) == ESHAPE
    assert L.fp8_weight_quant_block_ue8m0(P, 64, 128, P, P, None) == ESHAPE
    f = L.fp8_gemm_blockscaled_ue8m0
    assert f(None, P, P, P, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, P, P, P, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(PU, P, P, P, P, 4, 128, 128, None, 0, None) == EALIGN


def test_tensorscaled_gemm_argument_errors(L):
    f = L.fp8_gemm_tensorscaled
    assert f(None, P, P, P, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, None, P, P, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, P, P, P, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(P, P, P, P, PU, 4, 128, 128, None, 0, None) == EALIGN


def test_act_quant_gemm_argument_errors(L):
    f = L.fp8_act_quant_gemm_blockscaled
    ws = L.fp8_act_quant_gemm_blockscaled_workspace_bytes
    assert f(None, P, P, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, None, P, 4, 128, 128, None, 0, None) == ENULL
    assert f(P, P, P, P, 0, 128, 128, None, 0, None) == ESHAPE
    assert f(P, P, P, P, 4, 100, 128, None, 0, None) == ESHAPE
    assert f(P, P, P, P, 4, 128, 130, None, 0, None) == ESHAPE
    assert f(PU, P, P, P, 4, 128, 128, None, 0, None) == EALIGN
    assert f(P, P, P, PU, 4, 128, 128, None, 0, None) == EALIGN
    # one kernel (no workspace) for M <= 8 while x's codes and scales fit in LDS
    assert ws(1, 2048, 7168) == 0 and ws(4, 2048, 35712) == 0 and ws(8, 2048, 7168) == 0
    assert ws(8, 2048, 17792) == 0
    # otherwise act-quant and GEMM through the workspace: codes, scales, GEMM workspace
    assert ws(4, 2048, 35840) == 4 * 35840 + 4608
    assert ws(9, 2048, 7168) == 9 * 7168 + 2048
    assert ws(8, 2048, 17920) == 8 * 17920 + 4608
    assert ws(16, 2048, 7168) == 16 * 7168 + 3584
    assert ws(64, 2048, 7168) == 64 * 7168 + 14336 + L.fp8_gemm_blockscaled_workspace_bytes(64, 2048, 7168)
    assert ws(4096, 4096, 7168) == 4096 * 7168 + 4096 * 56 * 4
    assert f(P, P, P, P, 17, 128, 128, None, 0, None) == EWS
    assert f(P, P, P, P, 17, 128, 128, P, ws(17, 128, 128) - 1, None) == EWS


def test_act_quant_block_tensor_argument_errors(L):
    f = L.fp8_act_quant_block_tensor
    ws = L.fp8_act_quant_block_tensor_workspace_bytes
    assert ws(16384, 2048) == 16384 * 16 * 8 // 1024 * 4
    assert ws(1, 128) == 256 and ws(0, 128) == 0 and ws(4, 100) == 0
    assert f(None, 4, 128, P, P, P, P, P, 256, None) == ENULL
    assert f(P, 4, 128, P, P, None, P, P, 256, None) == ENULL
    assert f(P, 4, 100, P, P, P, P, P, 256, None) == ESHAPE
    assert f(P, 0, 128, P, P, P, P, P, 256, None) == ESHAPE
    assert f(PU, 4, 128, P, P, P, P, P, 256, None) == EALIGN
    assert f(P, 4, 128, P, P, PU, P, P, 256, None) == EALIGN
    assert f(P, 4, 128, P, P, P, P, None, 0, None) == EWS
    assert f(P, 4, 128, P, P, P, P, P, 255, None) == EWS
