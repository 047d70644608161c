#!/usr/bin/env python3
"""Benchmark of the FP8 quantize-and-multiply path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5|c4|c3|c2|c1] [--M m]
                    [--graph] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic input, with
the inputs resident in HBM before timing starts. Default workload (c5, the
large-M stress case M=16384, N=7168, K=2048): 1x128 block act-quant of A,
per-tensor amax quant of A, block-scaled FP8 GEMM with bf16 output. Other
workloads: c4 prefill (act-quant + GEMM, 4096x4096x7168), c3 decode (M tokens,
N=2048, K=7168), c2 per-tensor sweep (K=2048), c1 tiny (32x512x512).

Prints ONE JSON line. ``value`` is the step throughput expressed as GEMM
TFLOP/s (2*M*N*K per step / step time; per-tensor-only workloads use GB/s).
The default run also times every other workload the same way and reports
them under ``configs`` (c1; c2 per M with the amax stage alone beside the
TensorRT-LLM page's B200 figures; c3 per M as two calls and as the fused
call; c4); --no-sweep leaves that out.
The per-stage times come from HIP events around back-to-back launches of
each stage alone on the launch stream (replayed from a graph of their own
under --graph); ``roofline`` is for the dominant kernel. ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="c5", choices=["c5", "c4", "c3", "c2", "c1", "aq32", "copy"],
                   help="copy: a plain 256 MiB device-to-device copy (HBM reference for counters); "
                        "aq32: block act-quant of the prefill activation given as float32")
    p.add_argument("--M", type=int, default=None, help="rows for c2/c3")
    p.add_argument("--graph", dest="graph", action="store_true", default=True,
                   help="replay the steps from a HIP graph (the default)")
    p.add_argument("--no-graph", dest="graph", action="store_false",
                   help="launch every step from the host instead of replaying a graph")
    p.add_argument("--rotate", type=int, default=0,
                   help="input copies rotated across steps (0: enough copies for >= 512 MiB of distinct "
                        "inputs, twice the last-level cache, capped at 64)")
    p.add_argument("--scale-fmt", default="fp32", choices=["fp32", "ue8m0", "tensor"],
                   help="block scales: amax/448 (fp32) or powers of two (ue8m0: act-quant and weight quant "
                        "with power-of-two scales, GEMM with the matrix cores applying them); tensor: "
                        "one scale per tensor (per-tensor quant of A, then the per-tensor-scaled GEMM)")
    p.add_argument("--fused", action="store_true",
                   help="one call per step: block act-quant fused into the GEMM (fp8_act_quant_gemm_blockscaled)")
    p.add_argument("--separate-quant", action="store_true",
                   help="large-M workload: block and per-tensor quant as two calls (default: one call)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-sweep", dest="sweep", action="store_false", default=True,
                   help="default large-M run only: leave out the other workloads' figures (key 'configs')")
    p.add_argument("--cpu-rows", type=int, default=None, help="rows of the CPU oracle sample")
    return p.parse_args()


def src_hash(name):
    with open(os.path.join(ROOT, "fp8_block_scaled_act_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_key, src):
    """Bytes per launch between the L2 and the memory fabric (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings) from committed rocprofv3
    counter runs: what HBM or the last-level cache served, an upper bound on
    HBM bytes. None if the kernel source changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("src_sha256_16") != src_hash(src):
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads: synthetic inputs -> device tensors, and the per-stage launches

class Workload:
    def __init__(self, args, torch, fb):
        import synth
        self.torch, self.fb = torch, fb
        dev = "cuda:0"
        w = args.workload
        self.name = w
        self.stages = []          # (name, fn(i) -> None, algorithmic bytes, flops): one step
        self.extra = []           # stages timed on their own only (not part of a step)

        def rotation(per_copy_bytes):
            # cache honesty: the copies a stage cycles through span at least
            # 512 MiB (twice the 256 MiB last-level cache), so that timed
            # reads come from HBM; tiny inputs are capped (they are latency-bound)
            if args.rotate > 0:
                return args.rotate
            return int(min(64, max(2, -(-(512 << 20) // max(1, per_copy_bytes)))))

        def bf16(bits):
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
            return t.to(dev)

        if w == "copy":
            nbytes = 256 << 20
            src = torch.empty((nbytes,), dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            self.stages.append(("copy", lambda i: dst.copy_(src), 2 * nbytes, 0))
            self.config = {"workload": "plain device copy, 256 MiB", "bytes": nbytes}
            self.rot = 1
            self.M, self.N, self.K = nbytes, 0, 0
            self.cpu = None
            return

        if w == "c2":
            M = args.M or 65536
            K = 2048
            x = bf16(synth.gen_c2(M)["x"])
            rot = self.rot = rotation(2 * M * K)
            xs = [x] + [x.clone() for _ in range(rot - 1)]
            numel = M * K
            q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            s = torch.empty((1,), dtype=torch.float32, device=dev)
            wsb = fb.fp8_amax_quant_tensor_workspace_bytes(numel)
            ws = torch.zeros((max(wsb, 16),), dtype=torch.uint8, device=dev)
            self.stages.append(("amax_quant_tensor",
                                lambda i: fb.fp8_amax_quant_tensor(xs[i % rot], out=(q, s), workspace=ws),
                                3 * numel + 4, 0))
            amax = torch.empty((1,), dtype=torch.float32, device=dev)
            sa_only = torch.empty((1,), dtype=torch.float32, device=dev)
            self.extra.append(("amax_tensor",
                               lambda i: fb.fp8_amax_tensor(xs[i % rot], out=(amax, sa_only), workspace=ws),
                               2 * numel + 8, 0))
            # the apply step alone, with the dynamic op's scale given (on the device)
            fb.fp8_amax_quant_tensor(x, out=(q, s), workspace=ws)
            s_given = s.clone()
            self.extra.append(("static_quant_tensor",
                               lambda i: fb.fp8_static_quant_tensor(xs[i % rot], s_given, out=q),
                               3 * numel + 4, 0))
            self.config = {"workload": f"per-tensor dynamic quant, X bf16 [{M}, {K}]", "M": M, "K": K}
            self.M, self.N, self.K = M, 0, K
            self.cpu = ("c2", M, K, None)
            return

        if w == "aq32":
            M, K = 4096, 7168
            xf = torch.from_numpy(synth.bf16_bits_to_f64(synth.gen_c4()["a"]).astype(np.float32)).to(dev)
            rot = self.rot = rotation(4 * M * K)
            xs = [xf] + [xf.clone() for _ in range(rot - 1)]
            q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            s = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
            self.stages.append(("act_quant_block_f32",
                                lambda i: fb.fp8_act_quant_block_f32(xs[i % rot], out=(q, s)),
                                4 * M * K + M * K + 4 * (M * K // 128), 0))
            self.config = {"workload": f"block act-quant of float32 X [{M}, {K}]", "M": M, "K": K}
            self.M, self.N, self.K = M, 0, K
            self.cpu = ("aq32", M, K, None)
            return

        if w == "c1":
            d = synth.gen_c1(); M, N, K = 32, 512, 512
            wl = "tiny block quant + GEMM, A [32,512], W [512,512]"
        elif w == "c3":
            M = args.M or 64
            d = synth.gen_c3(M); N, K = 2048, 7168
            wl = f"decode block-scaled GEMM, M={M}, N=2048, K=7168"
        elif w == "c4":
            d = synth.gen_c4(); M, N, K = 4096, 4096, 7168
            wl = "prefill block-scaled GEMM, M=4096, N=4096, K=7168"
        else:
            d = synth.gen_c5(); M, N, K = 16384, 7168, 2048
            wl = "large-M stress: block act-quant + per-tensor quant + block-scaled GEMM, M=16384, N=7168, K=2048"
        self.M, self.N, self.K = M, N, K
        rot = self.rot = rotation(2 * M * K + N * K)
        a = bf16(d["a"])
        if args.scale_fmt == "tensor":
            wq, wsc = fb.fp8_amax_quant_tensor(bf16(d["w"]))
            a_s = [a] + [a.clone() for _ in range(rot - 1)]
            w_s = [wq] + [wq.clone() for _ in range(rot - 1)]
            qa = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(rot)]
            sa = [torch.empty((1,), dtype=torch.float32, device=dev) for _ in range(rot)]
            twsb = fb.fp8_amax_quant_tensor_workspace_bytes(M * K)
            tws = torch.zeros((max(twsb, 16),), dtype=torch.uint8, device=dev)
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            gwsb = fb.fp8_gemm_blockscaled_workspace_bytes(M, N, K)
            gws = torch.empty((max(gwsb, 16),), dtype=torch.uint8, device=dev)
            self.stages.append(("amax_quant_tensor",
                                lambda i: fb.fp8_amax_quant_tensor(a_s[i % rot], out=(qa[i % rot], sa[i % rot]),
                                                                   workspace=tws),
                                3 * M * K + 4, 0))
            self.stages.append(("gemm_blockscaled",
                                lambda i: fb.fp8_gemm_tensorscaled(qa[i % rot], sa[i % rot], w_s[i % rot], wsc,
                                                                   out=c, workspace=gws),
                                M * K + N * K + 8 + 2 * M * N, 2 * M * N * K))
            wl += " (one scale per tensor: per-tensor quant of A, per-tensor-scaled GEMM)"
            self.config = {"workload": wl, "M": M, "N": N, "K": K}
            self.cpu = None
            return
        if args.fused:
            if args.scale_fmt != "fp32" or w == "c5":
                raise SystemExit("--fused takes fp32 block scales and one of c1, c3, c4")
            wq, wsc = fb.fp8_weight_quant_block(bf16(d["w"]))
            a_s = [a] + [a.clone() for _ in range(rot - 1)]
            w_s = [wq] + [wq.clone() for _ in range(rot - 1)]
            c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fwsb = fb.fp8_act_quant_gemm_blockscaled_workspace_bytes(M, N, K)
            fws = torch.empty((max(fwsb, 16),), dtype=torch.uint8, device=dev)
            self.stages.append(("act_quant_gemm_blockscaled",
                                lambda i: fb.fp8_act_quant_gemm_blockscaled(a_s[i % rot], w_s[i % rot], wsc,
                                                                            out=c, workspace=fws),
                                2 * M * K + N * K + 4 * (N // 128) * (K // 128) + 2 * M * N, 2 * M * N * K))
            wl += " (block act-quant fused into the GEMM call)"
            self.config = {"workload": wl, "M": M, "N": N, "K": K}
            self.cpu = (w, M, K, N)
            return
        ue = args.scale_fmt == "ue8m0"
        act_q = fb.fp8_act_quant_block_ue8m0 if ue else fb.fp8_act_quant_block
        gemm_f = fb.fp8_gemm_blockscaled_ue8m0 if ue else fb.fp8_gemm_blockscaled
        wq, wsc = (fb.fp8_weight_quant_block_ue8m0 if ue else fb.fp8_weight_quant_block)(bf16(d["w"]))
        if "w_scale" in d:
            ws_host = d["w_scale"]
            if ue:   # the drawn scales, rounded up to powers of two
                ws_host = np.ldexp(np.float32(1.0), np.ceil(np.log2(ws_host)).astype(np.int32)).astype(np.float32)
            wsc = torch.from_numpy(ws_host).to(dev)
        a_s = [a] + [a.clone() for _ in range(rot - 1)]
        w_s = [wq] + [wq.clone() for _ in range(rot - 1)]
        qa = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(rot)]
        sa = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(rot)]
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        gwsb = fb.fp8_gemm_blockscaled_workspace_bytes(M, N, K)
        gws = torch.empty((max(gwsb, 16),), dtype=torch.uint8, device=dev)
        fuse_bt = w == "c5" and not ue and not args.separate_quant
        if fuse_bt:
            # block and per-tensor quant of A in one call (A read twice, not three times)
            qt = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            st = torch.empty((1,), dtype=torch.float32, device=dev)
            bwsb = fb.fp8_act_quant_block_tensor_workspace_bytes(M, K)
            bws = torch.zeros((max(bwsb, 16),), dtype=torch.uint8, device=dev)
            self.stages.append(("act_quant_block_tensor",
                                lambda i: fb.fp8_act_quant_block_tensor(
                                    a_s[i % rot], out=(qa[i % rot], sa[i % rot], qt, st), workspace=bws),
                                2 * M * K + 2 * M * K + 4 * (M * K // 128) + 4, 0))
        else:
            self.stages.append(("act_quant_block",
                                lambda i: act_q(a_s[i % rot], out=(qa[i % rot], sa[i % rot])),
                                2 * M * K + M * K + 4 * (M * K // 128), 0))
        if w == "c5" and not fuse_bt:
            qt = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
            st = torch.empty((1,), dtype=torch.float32, device=dev)
            twsb = fb.fp8_amax_quant_tensor_workspace_bytes(M * K)
            tws = torch.zeros((max(twsb, 16),), dtype=torch.uint8, device=dev)
            self.stages.append(("amax_quant_tensor",
                                lambda i: fb.fp8_amax_quant_tensor(a_s[i % rot], out=(qt, st), workspace=tws),
                                3 * M * K + 4, 0))
        gemm_bytes = M * K + 4 * M * (K // 128) + N * K + 4 * (N // 128) * (K // 128) + 2 * M * N
        self.stages.append(("gemm_blockscaled",
                            lambda i: gemm_f(qa[i % rot], sa[i % rot], w_s[i % rot], wsc,
                                             out=c, workspace=gws),
                            gemm_bytes, 2 * M * N * K))
        if fuse_bt:
            wl += " (block and per-tensor quant of A in one call)"
        if ue:
            wl += " (power-of-two block scales)"
        self.config = {"workload": wl, "M": M, "N": N, "K": K}
        self.cpu = (w, M, K, N)


def time_steps(torch, wl, steps, warmup, graph):
    """Warm up, then time exactly `steps` steps between two HIP events on the
    launch stream (torch's current stream, where the library enqueues); one
    more untimed step is queued just before the start event so that the host's
    launch of the timed steps does not leave the GPU idle inside the timed
    region (the region still holds exactly `steps` steps). Then,
    for the per-stage figures, time `steps` back-to-back launches of each
    stage alone the same way (average duration per launch), after a pass that
    gives the spread: each launch between its own pair of events, or, with
    graphs, ten replays of the stage's graph."""
    st = torch.cuda.current_stream()
    for i in range(warmup):
        for _, fn, _, _ in wl.stages:
            fn(i)
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(st)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for i in range(steps):
                    for _, fn, _, _ in wl.stages:
                        fn(i)
        torch.cuda.synchronize()
        g.replay()                                       # one untimed replay
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # the last warm-up step is queued right before the start event, so that
    # the GPU is busy while the host launches the timed steps (a graph launch
    # takes the host a few hundred microseconds before its first kernel runs)
    for _, fn, _, _ in wl.stages:
        fn(warmup)
    e0, e1 = ev(), ev()
    e0.record(st)
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            for _, fn, _, _ in wl.stages:
                fn(warmup + 1 + i)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps

    per_stage = []
    for _, fn, _, _ in wl.stages + wl.extra:
        gs = None
        if graph:
            # the stage's launches alone, replayed from a graph of their own
            gs = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(st)
            with torch.cuda.stream(cs):
                with torch.cuda.graph(gs, stream=cs):
                    for i in range(steps):
                        fn(i)
            torch.cuda.synchronize()
            gs.replay()
            torch.cuda.synchronize()
        # spread (median, p10, p90 of per-launch times)
        if gs is not None:
            reps = []
            for _ in range(10):
                fn(0)                      # queued in front, as for the steps
                a, b = ev(), ev()
                a.record(st)
                gs.replay()
                b.record(st)
                torch.cuda.synchronize()
                reps.append(a.elapsed_time(b) / steps)
        else:
            evs = [ev() for _ in range(steps + 1)]
            evs[0].record(st)
            for i in range(steps):
                fn(i)
                evs[i + 1].record(st)
            torch.cuda.synchronize()
            reps = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        spread = (float(np.median(reps)), float(np.percentile(reps, 10)), float(np.percentile(reps, 90)))
        # the average: back-to-back launches between one pair of events
        fn(0)
        a, b = ev(), ev()
        a.record(st)
        if gs is not None:
            gs.replay()
        else:
            for i in range(steps):
                fn(i)
        b.record(st)
        torch.cuda.synchronize()
        per_stage.append((a.elapsed_time(b) / steps, spread))
    return step_ms, per_stage, wall


def cpu_baseline(wl, rows_arg, ue8m0=False):
    """The oracle, as it stands, on a bounded row sample of the same workload."""
    import synth
    from oracle import gemm as ogemm, quant as oquant
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    kind, M, K, N = wl.cpu
    t = 0.0
    if kind == "aq32":
        rows = min(M, rows_arg or 1024)
        x = synth.bf16_bits_to_f64(synth.gen_c4()["a"][:rows]).astype(np.float32)
        t0 = time.perf_counter(); oquant.act_quant_block_f32(x); t = time.perf_counter() - t0
        value = (5 * rows * K + 4 * rows * (K // 128)) / t / 1e9
        return {"value": value, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"block quant of float32 [{rows}, {K}] (numpy, one thread), {t:.2f} s"}
    if kind == "c2":
        rows = min(M, rows_arg or M)
        x = synth.gen_c2(rows)["x"]
        t0 = time.perf_counter(); oquant.amax_quant_tensor(x); t = time.perf_counter() - t0
        value = (3 * rows * K + 4) / t / 1e9
        return {"value": value, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"per-tensor quant of [{rows}, {K}] bf16 (numpy, one thread), {t:.2f} s"}
    rows = min(M, rows_arg or M)
    d = {"c1": lambda: synth.gen_c1(), "c3": lambda: synth.gen_c3(M), "c4": lambda: synth.gen_c4(),
         "c5": lambda: synth.gen_c5()}[kind]()
    a = d["a"][:rows]
    qw, sw = (oquant.weight_quant_block_ue8m0 if ue8m0 else oquant.weight_quant_block)(d["w"])  # offline
    if "w_scale" in d:
        sw = d["w_scale"]
    t0 = time.perf_counter()
    qa, sa = (oquant.act_quant_block_ue8m0 if ue8m0 else oquant.act_quant_block)(a)
    if kind == "c5":
        oquant.amax_quant_tensor(a)
    ogemm.gemm_blockscaled_ref(qa, sa, qw, sw)
    t = time.perf_counter() - t0
    value = 2.0 * rows * N * K / t / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": (f"rows 0..{rows - 1} of A ({rows} of {M}): block quant"
                       + (" + per-tensor quant" if kind == "c5" else "")
                       + f" (numpy, one thread) + fp64 GEMM {rows}x{N}x{K} (BLAS, {blas_threads} threads); "
                       f"{t:.2f} s; value = 2*rows*N*K / time")}


def summarize(wl, per_stage, scale_fmt="fp32", workload_key=None):
    """Per-stage figures (us per launch, spread, GB/s and TFLOP/s with their
    roofline fractions) and the roofline object of the dominant kernel."""
    stages = {}
    for j, (name, _, nbytes, flops) in enumerate(wl.stages + wl.extra):
        e = {"algorithmic_bytes": nbytes}
        avg_ms, (med, p10, p90) = per_stage[j]
        us = float(avg_ms) * 1e3
        e["us_per_launch"] = us
        e["us_median"], e["us_p10"], e["us_p90"] = med * 1e3, p10 * 1e3, p90 * 1e3
        e["GB/s"] = nbytes / (us * 1e-6) / 1e9
        e["hbm_frac"] = e["GB/s"] / HBM_PEAK_GBS
        if flops:
            e["TFLOP/s"] = flops / (us * 1e-6) / 1e12
            e["mfma_frac"] = e["TFLOP/s"] / FP8_PEAK_TFLOPS
        stages[name] = e
    # dominant kernel: the GEMM when present (prefill: MFMA-bound; decode: HBM-bound)
    if "gemm_blockscaled" in stages:
        dominant = "gemm_blockscaled"
    elif "act_quant_gemm_blockscaled" in stages:
        dominant = "act_quant_gemm_blockscaled"
    else:
        dominant = wl.stages[0][0]
    ds = stages[dominant]
    src = "gemm.hip" if "gemm" in dominant else "quant.hip"
    fmt = "_ue8m0" if scale_fmt == "ue8m0" and dominant != "amax_quant_tensor" else ""
    traffic = load_traffic(f"{dominant}{fmt}:{workload_key or wl.name}", src)
    if "gemm" in dominant and 2 * wl.M * wl.N * wl.K / max(ds["algorithmic_bytes"], 1) > 625:
        roofline = {"bound": "mfma", "achieved": ds["TFLOP/s"], "peak": FP8_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": ds["TFLOP/s"] / FP8_PEAK_TFLOPS, "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "achieved": ds["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": ds["GB/s"] / HBM_PEAK_GBS, "traffic": traffic}
    roofline["kernel"] = dominant
    roofline["us_per_launch"] = ds["us_per_launch"]
    return stages, roofline


# the TensorRT-LLM page's B200 amax-stage times (section "Test Coverage", the
# fixed design, under CUDA graph), per M at K = 2048: context, not a target
B200_AMAX_US = {1: 4.1, 64: 4.1, 256: 6.1, 1024: 6.1, 65536: 43.0}


def sweep(torch, fb, steps, warmup, graph):
    """Every other workload, timed the same way (inputs resident, rotated,
    stages replayed from graphs): us per call, GB/s or TFLOP/s and the
    roofline fraction of each stage, and the step time."""
    from types import SimpleNamespace

    def one(workload, M=None, fused=False):
        spec = SimpleNamespace(workload=workload, M=M, rotate=0, scale_fmt="fp32", fused=fused,
                               separate_quant=False)
        wl = Workload(spec, torch, fb)
        ms, per_stage, _ = time_steps(torch, wl, steps, warmup, graph)
        stages, roofline = summarize(wl, per_stage, workload_key=workload)
        keep = ("us_per_launch", "us_median", "GB/s", "hbm_frac", "TFLOP/s", "mfma_frac")
        out = {"step_us": ms * 1e3,
               "stages": {k: {f: round(v[f], 4) for f in keep if f in v} for k, v in stages.items()},
               "roofline": {k: roofline[k] for k in ("kernel", "bound", "achieved", "unit", "frac")},
               "rotated_copies": wl.rot}
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        return out

    res = {"c1": one("c1")}
    c2 = {}
    for M in (1, 64, 256, 1024, 65536):
        r = one("c2", M)
        r["b200_amax_us_context"] = B200_AMAX_US[M]
        c2[f"M={M}"] = r
    res["c2"] = c2
    res["c3"] = {f"M={M}": {"two_calls": one("c3", M), "fused_call": one("c3", M, fused=True)}
                 for M in (1, 8, 32, 64)}
    res["c4"] = one("c4")
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    import fp8_block_scaled_act_amd as fb
    fb.lib()
    torch.cuda.set_device(0)
    wl = Workload(args, torch, fb)
    ms, per_stage, wall = time_steps(torch, wl, args.steps, args.warmup, args.graph)
    stages, roofline = summarize(wl, per_stage, args.scale_fmt, args.workload)
    wl_config, wl_rot = wl.config, getattr(wl, "rot", 1)

    if wl.N:
        value = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        value = wl.stages[0][2] / (ms * 1e-3) / 1e9
        unit = "GB/s"

    cpu = None
    if not args.no_cpu_baseline and wl.cpu is not None:
        cpu = cpu_baseline(wl, args.cpu_rows, ue8m0=args.scale_fmt == "ue8m0")
        cpu["host_cpus"] = os.cpu_count()
        try:
            cpu["affinity_cpus"] = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            pass

    configs = None
    if args.sweep and args.workload == "c5" and args.scale_fmt == "fp32" and not args.separate_quant:
        del wl
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        configs = sweep(torch, fb, min(args.steps, 50), min(args.warmup, 10), args.graph)

    line = {
        "metric": "FP8 block-scaled GEMM TFLOP/s + act-quant GB/s (%roofline), 1 MI355X",
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate, bf16 in/out)",
        "data": "synthetic (seeded numpy generators; inputs resident in HBM, "
                f"{wl_rot} rotated input copies"
                + (", >= 512 MiB of distinct inputs)" if args.rotate == 0 else ")"),
        "config": None,
        "timing": ("step: HIP events around all steps" + (" (HIP graph replay)" if args.graph else "")
                   + ", the last warm-up step queued just before the start event"
                   + "; stages: HIP events around back-to-back launches of each stage"
                   + (" (each stage replayed from a graph of its own)" if args.graph else "")
                   + "; us_median/p10/p90: " + ("over ten replays of the stage's graph" if args.graph
                                               else "each launch between its own pair of events")),
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed_region": wall,
    }
    line["config"] = wl_config
    if configs is not None:
        line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
