"""Entry points replayed from a captured HIP graph (torch.cuda.CUDAGraph), the
way a serving loop (and bench.py) runs them.

Each case captures one call on fixed input buffers, then replays the graph
several times. Between replays, eager work writes new inputs into the
captured buffers, and the host synchronizes. Every replay must equal, bit for
bit, the eager call on the same inputs. This covers the multi-launch paths
as well: the per-tensor quant's two passes, the split-K GEMM with its reduce
kernel, and the fused act-quant + GEMM in both of its forms.
"""
import pytest
import torch

from tests.helpers import binding, say

pytestmark = pytest.mark.gpu

REPLAYS = 4


def bf16(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device="cuda:0") * scale).to(torch.bfloat16)


def as_list(out):
    return list(out) if isinstance(out, (tuple, list)) else [out]


def same_bits(a, b):
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def replay_matches_eager(label, make_inputs, call):
    """make_inputs(r) -> list of input tensors for round r; call(*inputs) ->
    tensor or tuple of tensors."""
    static = [t.clone() for t in make_inputs(0)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(*static)                              # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = as_list(call(*static))
    for r in range(1, REPLAYS + 1):
        say("graph replay", label, "round", r)
        fresh = make_inputs(r)
        for dst, src in zip(static, fresh):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = as_list(call(*fresh))
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(got, want)):
            assert same_bits(a, b), (label, r, k)


@pytest.mark.parametrize("M,K", [(1, 7168), (64, 7168), (4096, 2048)])
def test_act_quant_block(M, K):
    fb = binding()
    replay_matches_eager(f"act_quant_block {M}x{K}", lambda r: [bf16((M, K), 100 + r, 3.0)],
                         fb.fp8_act_quant_block)


@pytest.mark.parametrize("M,K", [(1, 2048), (1024, 2048), (65536, 2048)])
def test_amax_quant_tensor(M, K):
    fb = binding()
    # the scale changes from round to round, so a stale partial maximum shows
    replay_matches_eager(f"amax_quant_tensor {M}x{K}", lambda r: [bf16((M, K), 200 + r, 1.0 + r)],
                         fb.fp8_amax_quant_tensor)


def test_act_quant_block_tensor():
    fb = binding()
    M, K = 2048, 2048
    replay_matches_eager("act_quant_block_tensor", lambda r: [bf16((M, K), 300 + r, 1.0 + r)],
                         fb.fp8_act_quant_block_tensor)


def gemm_inputs(fb, M, N, K, r, quant=None):
    quant = quant or fb.fp8_act_quant_block
    qa, sa = quant(bf16((M, K), 400 + r, 2.0))
    qw, sw = fb.fp8_weight_quant_block(bf16((N, K), 500 + r, 0.02))
    return [qa, sa, qw, sw]


# decode M = 1 (packed K blocks), 12, 40 and 64 at N = 2048 (chunked full-K
# kernel), 40 and 64 at N = 4096 (split-K with the reduce kernel); M = 300
# (tiled kernel with K split, and its reduce) and 2048 (tiled kernel)
@pytest.mark.parametrize("M,N,K", [(1, 2048, 7168), (12, 2048, 7168), (40, 2048, 7168), (64, 2048, 7168),
                                   (40, 4096, 2048), (64, 4096, 7168), (300, 1024, 2048), (2048, 2048, 2048)])
def test_gemm_blockscaled(M, N, K):
    fb = binding()
    replay_matches_eager(f"gemm_blockscaled {M}x{N}x{K}", lambda r: gemm_inputs(fb, M, N, K, r),
                         fb.fp8_gemm_blockscaled)


@pytest.mark.parametrize("M,N,K", [(40, 2048, 7168), (40, 4096, 2048), (2048, 2048, 2048)])
def test_gemm_ue8m0(M, N, K):
    fb = binding()

    def inputs(r):
        qa, sa = fb.fp8_act_quant_block_ue8m0(bf16((M, K), 600 + r, 2.0))
        qw, sw = fb.fp8_weight_quant_block_ue8m0(bf16((N, K), 700 + r, 0.02))
        return [qa, sa, qw, sw]

    replay_matches_eager(f"gemm_ue8m0 {M}x{N}x{K}", inputs, fb.fp8_gemm_blockscaled_ue8m0)


@pytest.mark.parametrize("M,N,K", [(40, 2048, 7168), (40, 4096, 2048), (2048, 2048, 2048)])
def test_gemm_tensorscaled(M, N, K):
    fb = binding()

    def inputs(r):
        qa, sa = fb.fp8_amax_quant_tensor(bf16((M, K), 800 + r, 2.0))
        qw, sw = fb.fp8_amax_quant_tensor(bf16((N, K), 900 + r, 0.02))
        return [qa, sa, qw, sw]

    replay_matches_eager(f"gemm_tensorscaled {M}x{N}x{K}", inputs, fb.fp8_gemm_tensorscaled)


# M = 2: one kernel; M = 8 and 48 at N = 2048: act-quant and GEMM through the
# workspace; M = 48 at N = 4096: act-quant, split-K GEMM and its reduce
@pytest.mark.parametrize("M,N", [(2, 2048), (8, 2048), (48, 2048), (48, 4096)])
def test_act_quant_gemm(M, N):
    fb = binding()
    K = 7168

    def inputs(r):
        qw, sw = fb.fp8_weight_quant_block(bf16((N, K), 1000 + r, 0.02))
        return [bf16((M, K), 1100 + r, 2.0), qw, sw]

    replay_matches_eager(f"act_quant_gemm M={M}", inputs, fb.fp8_act_quant_gemm_blockscaled)
