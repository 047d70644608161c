"""The C ABI from several host threads at once, each on its own HIP stream:
the library keeps no mutable state besides its per-device cache, so every
thread's results must equal, bit for bit, the same calls made one after the
other. Each thread owns its outputs and workspaces."""
import threading

import numpy as np
import pytest
import torch

import synth
from tests.helpers import bf16_to_dev, binding, say, to_bf16_bits, to_f32, to_u8

pytestmark = pytest.mark.gpu


def pipeline(fb, x, qw, sw, stream):
    with torch.cuda.stream(stream):
        qa, sa = fb.fp8_act_quant_block(x)
        c = fb.fp8_gemm_blockscaled(qa, sa, qw, sw)
        qt, st = fb.fp8_amax_quant_tensor(x)
        cf = fb.fp8_act_quant_gemm_blockscaled(x[:4].contiguous(), qw, sw)
    return qa, sa, c, qt, st, cf


def host(outs):
    return [to_u8(outs[0]), to_f32(outs[1]).view(np.uint32), to_bf16_bits(outs[2]), to_u8(outs[3]),
            to_f32(outs[4]).view(np.uint32), to_bf16_bits(outs[5])]


def test_threads_on_their_own_streams_match_sequential_calls():
    fb = binding()
    rng = np.random.default_rng(77)
    shapes = [(96, 512, 1024), (40, 256, 2048), (300, 384, 512), (8, 640, 1536)]
    inputs = []
    for M, N, K in shapes:
        x = bf16_to_dev(synth.f64_to_bf16_bits(rng.standard_normal((M, K)) * 2))
        qw, sw = fb.fp8_weight_quant_block(bf16_to_dev(synth.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)))
        inputs.append((x, qw, sw))
    torch.cuda.synchronize()
    say("sequential reference", shapes)
    ref = []
    for x, qw, sw in inputs:
        s = torch.cuda.Stream()
        outs = pipeline(fb, x, qw, sw, s)
        s.synchronize()
        ref.append(host(outs))

    results = [None] * len(inputs)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            got = None
            for _ in range(3):                      # several rounds, overlapping the other threads
                got = pipeline(fb, *inputs[i], s)
            s.synchronize()
            results[i] = host(got)
        except Exception as e:                      # reported after the join
            errors.append((i, repr(e)))

    say("four threads, own streams")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for i, (r, g) in enumerate(zip(ref, results)):
        for k, (a, b) in enumerate(zip(r, g)):
            assert np.array_equal(a, b), (shapes[i], k)
