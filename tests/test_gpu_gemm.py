"""GPU parity of the block-scaled FP8 GEMM against the fp64 oracle over the
dequantized operands, through the C ABI.

Operands are quantized by the oracle (never by the GPU). The comparison rule
(oracle.gemm.compare_gemm): normwise max|C-R|/max|R| <= 1e-2 and elementwise
|C-R| <= 4 bf16 ulp(R) + the accumulation floor of FP8 matrix-core dot
products plus fp32 scaling and accumulation.
The integer-valued case is bit-exact: every fp32 partial sum is an exact
integer there, so any summation order gives bf16_rne(exact).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import e4m3, gemm, quant
from tests.helpers import (bf16_to_dev, binding, f32_to_dev, say, to_bf16_bits, u8_to_dev)

pytestmark = pytest.mark.gpu


def operands(a_bits, w_bits, w_scale=None):
    qa, sa = quant.act_quant_block(a_bits)
    qw, sw = quant.weight_quant_block(w_bits)
    if w_scale is not None:
        sw = np.asarray(w_scale, np.float32)
    return qa, sa, qw, sw


def run_gemm(qa, sa, qw, sw, label):
    fb = binding()
    say("gemm_blockscaled", label, qa.shape, qw.shape)
    c = fb.fp8_gemm_blockscaled(u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    torch.cuda.synchronize()
    return to_bf16_bits(c)


def check_full(qa, sa, qw, sw, label, c=None):
    if c is None:
        c = run_gemm(qa, sa, qw, sw, label)
    R = gemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    S = gemm.gemm_abs_ref(qa, sa, qw, sw)
    Se = gemm.gemm_exp_envelope_ref(qa, sa, qw, sw)
    res = gemm.compare_gemm(c, R, S, qa.shape[1], Se)
    assert res["ok"], (label, res)
    return res


def check_rows(qa, sa, qw, sw, rows, label):
    c = run_gemm(qa, sa, qw, sw, label)
    R = gemm.gemm_blockscaled_ref(qa[rows], sa[rows], qw, sw)
    S = gemm.gemm_abs_ref(qa[rows], sa[rows], qw, sw)
    Se = gemm.gemm_exp_envelope_ref(qa[rows], sa[rows], qw, sw)
    res = gemm.compare_gemm(c[rows], R, S, qa.shape[1], Se)
    assert res["ok"], (label, res)
    return res


def test_c1_tiny():
    d = synth.gen_c1()
    check_full(*operands(d["a"], d["w"]), "C1 32x512x512")


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_c3_decode(M):
    d = synth.gen_c3(M)
    check_full(*operands(d["a"], d["w"]), f"C3 M={M}")


def test_c4_prefill_sampled_rows():
    d = synth.gen_c4()
    qa, sa, qw, sw = operands(d["a"], d["w"])
    rows = np.sort(np.random.default_rng(44).choice(qa.shape[0], 192, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 127, 128, 4095]]))
    check_rows(qa, sa, qw, sw, rows, "C4 4096x4096x7168")


def test_large_tiles_ragged_k_blocks_sampled_rows():
    # enough 256 x 256 tiles to fill the chip, ragged M, and 13 K blocks: the
    # activation scales travel in chunks of 8 K blocks, the second one partial
    M, N, K = 4133, 4096, 1664
    rng = np.random.default_rng(4133)
    a = synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 2)
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa, sa, qw, sw = operands(a, w)
    rows = np.unique(np.concatenate([rng.choice(M, 96, replace=False), [0, 255, 256, 4095, 4096, 4132]]))
    check_rows(qa, sa, qw, sw, rows, f"{M}x{N}x{K}")


def test_c5_large_m_sampled_rows():
    d = synth.gen_c5()
    qa, sa, qw, sw = operands(d["a"], d["w"], d["w_scale"])
    kb = qa.shape[1] // 128
    special = np.concatenate([d["zero_blocks"][:16] // kb, d["big_blocks"][:16] // kb])
    rng = np.random.default_rng(55)
    rows = np.unique(np.concatenate([rng.choice(qa.shape[0], 160, replace=False), special,
                                     [0, 16383]]))
    check_rows(qa, sa, qw, sw, rows, "C5 16384x7168x2048")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (17, 256, 384), (129, 384, 256),
                                   (200, 128, 1024), (255, 512, 128), (300, 640, 640),
                                   (300, 384, 2432), (133, 256, 1152), (65, 256, 640)])
def test_ragged_shapes(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = synth.f64_to_bf16_bits(rng.standard_t(3.0, size=(M, K)))
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    sw = (10.0 ** rng.uniform(-4, -1, size=(N // 128, K // 128))).astype(np.float32)
    check_full(*operands(a, w, sw), f"ragged {M}x{N}x{K}")


INT_CODES = {0: 0x00, 1: 0x38, 2: 0x40, 3: 0x44, 4: 0x48}


def int_codes(vals):
    mag = np.vectorize(lambda v: INT_CODES[abs(int(v))])(vals).astype(np.uint8)
    return mag | np.where(vals < 0, 0x80, 0).astype(np.uint8)


@pytest.mark.parametrize("M,N,K", [(64, 256, 7168), (130, 384, 2048)])
def test_integer_valued_bit_exact(M, N, K):
    rng = np.random.default_rng(M * N)
    ia = rng.integers(-4, 5, size=(M, K))
    iw = rng.integers(-4, 5, size=(N, K))
    qa, qw = int_codes(ia), int_codes(iw)
    assert np.array_equal(e4m3.DECODE[qa], ia)
    sa = np.ones((M, K // 128), np.float32)
    sw = np.ones((N // 128, K // 128), np.float32)
    c = run_gemm(qa, sa, qw, sw, f"integer {M}x{N}x{K}")
    exact = (ia @ iw.T).astype(np.float64)
    assert np.max(np.abs(exact)) < 2 ** 24
    assert np.array_equal(c, gemm.f64_to_bf16_rne(exact))


def test_identity_weight():
    rng = np.random.default_rng(8)
    M, K = 96, 512
    qa, sa = quant.act_quant_block(synth.f64_to_bf16_bits(rng.standard_normal((M, K))))
    qw = np.zeros((K, K), np.uint8)
    np.fill_diagonal(qw, 0x38)
    sw = np.ones((K // 128, K // 128), np.float32)
    c = run_gemm(qa, sa, qw, sw, "identity")
    # C = bf16(dec(qa) * sa): one exact product (e4m3 x fp32 fits in fp32) rounded once
    want = gemm.f64_to_bf16_rne(gemm.dequant_act(qa, sa))
    assert np.array_equal(c, want)


def test_zero_scales_and_zero_blocks():
    rng = np.random.default_rng(9)
    M, N, K = 40, 256, 512
    a = rng.standard_normal((M, K))
    a[:, 128:256] = 0.0
    qa, sa = quant.act_quant_block(synth.f64_to_bf16_bits(a))
    qw, sw = quant.weight_quant_block(synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02))
    sw[1, :] = 0.0
    c = check_full(qa, sa, qw, sw, "zero scales")
    out = run_gemm(qa, sa, qw, sw, "zero scales again")
    assert np.all(out[:, 128:256] & 0x7FFF == 0)


def test_deterministic():
    fb = binding()
    d = synth.gen_c3(32)
    qa, sa, qw, sw = operands(d["a"], d["w"])
    args = (u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    c1 = fb.fp8_gemm_blockscaled(*args)
    c2 = fb.fp8_gemm_blockscaled(*args)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)


def model_gemm(qa, sa, qw, sw):
    """Bit-level model of the kernel's arithmetic: per K block the matrix-core
    dot product (tests/mfma_model.py), times the fp32 product sa*sw, added into
    an fp32 accumulator in K order; bf16 rounding at the end. Exact emulation
    when every scale is a power of two (then each scaled term is exact)."""
    from tests.mfma_model import block_dot
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.zeros((M, N), np.float32)
    for b in range(K // 128):
        P = block_dot(qa[:, None, b * 128:(b + 1) * 128], qw[None, :, b * 128:(b + 1) * 128])
        cs = (sa[:, b][:, None] * np.repeat(sw[:, b], 128)[None, :]).astype(np.float32)
        acc = (acc + (P * cs).astype(np.float32)).astype(np.float32)
    return gemm.f64_to_bf16_rne(acc.astype(np.float64))


@pytest.mark.parametrize("dist", ["uniform_codes", "normal", "cancel"])
def test_bit_exact_against_matrix_core_model(dist):
    rng = np.random.default_rng({"uniform_codes": 1, "normal": 2, "cancel": 3}[dist])
    M, N, K = 96, 256, 512
    fin = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    if dist == "uniform_codes":
        qa = rng.choice(fin, size=(M, K)); qw = rng.choice(fin, size=(N, K))
    else:
        qa = e4m3.encode(np.clip(rng.standard_normal((M, K)) * 60, -448, 448).astype(np.float32))
        qw = e4m3.encode(np.clip(rng.standard_normal((N, K)) * 60, -448, 448).astype(np.float32))
        if dist == "cancel":
            qw[: M] = qa ^ np.uint8(0x80)                 # rows n < M cancel row m = n
            qw[: M, ::5] = rng.choice(fin, size=(M, K // 5 + 1))[:, : qw[:, ::5].shape[1]]
    qa = qa.astype(np.uint8); qw = qw.astype(np.uint8)
    sa = np.ldexp(1.0, rng.integers(-6, 4, size=(M, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, rng.integers(-8, 2, size=(N // 128, K // 128))).astype(np.float32)
    c = run_gemm(qa, sa, qw, sw, f"matrix-core model {dist}")
    want = model_gemm(qa, sa, qw, sw)
    bad = np.argwhere(c != want)
    assert bad.shape[0] == 0, (dist, bad.shape[0], bad[:4].tolist())
    check_full(qa, sa, qw, sw, f"tolerance {dist}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 1024), (16, 2048, 7168), (17, 384, 2048),
                                   (33, 640, 4096), (64, 2048, 7168), (64, 128, 128 * 40), (48, 7168, 2048),
                                   (3, 256, 128 * 7), (16, 128, 128 * 600), (40, 128, 128 * 500),
                                   (2, 128, 71424), (2, 128, 71552), (13, 384, 128 * 9), (9, 128, 128)])
def test_decode_shapes(M, N, K):
    # M <= 16: sixteen waves per workgroup, each taking every sixteenth step
    # of K, partial sums added in a fixed order (K = 7 blocks leaves waves
    # without a step; K = 600 blocks runs many prefetch rounds per wave).
    # M <= 8 packs two K blocks into each MFMA (8 W rows per workgroup): an
    # odd block count (1, 7, 559) leaves the last step half empty. 8 < M <= 16
    # takes 8 W rows per workgroup too, the MFMA's other 8 rows zero.
    # 16 < M <= 64: several K splits, fp32 partials in the workspace, reduced
    # in split order.
    rng = np.random.default_rng(M * 7 + N + K)
    a = synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 3)
    w = synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    check_full(*operands(a, w), f"decode {M}x{N}x{K}")


def test_gemm_workspace_size_and_reuse():
    fb = binding()
    N, K = 2048, 7168
    for M in (1, 8, 16, 65, 4096):
        assert fb.fp8_gemm_blockscaled_workspace_bytes(M, N, K) == 0
    M = 32
    wsb = fb.fp8_gemm_blockscaled_workspace_bytes(M, N, K)
    assert wsb >= M * N * 4 and wsb % (M * N * 4) == 0    # fp32 partials, one [M, N] per K split
    d = synth.gen_c3(M)
    qa, sa, qw, sw = operands(d["a"], d["w"])
    args = (u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device="cuda:0")     # garbage on entry
    c1 = fb.fp8_gemm_blockscaled(*args, workspace=ws)
    c2 = fb.fp8_gemm_blockscaled(*args, workspace=ws)
    # other garbage: consecutive 64-bit integers
    ws_seq = torch.arange(wsb // 8, dtype=torch.int64, device="cuda:0").view(torch.uint8)
    c3 = fb.fp8_gemm_blockscaled(*args, workspace=ws_seq)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(c1, c3)
    check_full(qa, sa, qw, sw, "decode M=32 through a reused workspace", c=to_bf16_bits(c2))
    with pytest.raises(fb.Fp8bsError):
        fb.fp8_gemm_blockscaled(*args, workspace=ws[: wsb - 4])


@pytest.mark.parametrize("M", [1, 5, 8, 12, 16, 40])
def test_decode_paths_are_deterministic(M):
    # the decode kernels add their partial sums in a fixed order (waves, K
    # block groups, K splits), so repeated calls give identical bits
    fb = binding()
    d = synth.gen_c3(M)
    qa, sa, qw, sw = operands(d["a"], d["w"])
    args = (u8_to_dev(qa), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw))
    say("decode determinism", M)
    outs = [fb.fp8_gemm_blockscaled(*args) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:]), M
