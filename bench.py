"""Benchmark of the Q4_K linear layer on one MI355X.

One *step* is one pass of the whole hot path over the workload's synthetic
inputs, each kernel on cold weights:
  * decode GEMV, W 4096 x 4096 Q4_K, fp32 x (the headline configuration), and
    the same shape on the Q5_K, Q6_K and Q3_K sibling formats;
  * small-batch GEMV and GEMM, W 14336 x 4096, M in {1, 2, 4, 8, 16, 32};
  * SwiGLU MLP at one token: gate/up 14336 x 4096, down 4096 x 14336;
  * prefill GEMM, X bf16 [512, 4096], W 4096 x 4096 and 14336 x 4096;
  * the bf16 dequantization export of the 4096 x 4096 matrix;
  * the INT8 W8A8 linear layer at the xpu-kernels page's shape, K = N = 3072,
    M = 1024 (its headline row) and 8192: the row quantizer of the bf16
    activations and the int8 MFMA GEMM with the fused dequant epilogue.
Every kernel rotates over copies of its working set totalling >= 576 MB (past
the 256 MB MALL and the 4 MB L2 per XCD), so each launch reads cold HBM.

Timing: W warm-up steps, then K steps bracketed by a device synchronize.  The
K launches of one kernel run back to back on the launch stream between two
HIP events; the per-launch average is that kernel's duration (launch gaps
included) and the roofline figures use it.  Beside it, per kernel: the
per-dispatch device durations (median, p10, p90 of the K dispatches, from the
runtime's activity trace through torch.profiler -- the timestamps rocprofv3's
kernel trace reads) and the same K launches replayed from one HIP graph.
``value`` is the decode GEMV's effective HBM bandwidth (algorithmic bytes /
average duration).  The parity spot check reads the outputs of the last
launch.  The CPU baseline times the oracle on the host's cores (one thread and
all of them) on the decode GEMV, the MLP and the prefill GEMM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       [--only LIST] [--eager-only] [--no-dispatch-trace]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
INT8_PEAK_TOPS = 5033.2        # MI355X dense int8 MFMA (256 CU x 2.4 GHz x 8192 OP/clk)
COLD_BYTES = 576 << 20         # rotating working set per kernel: over twice the 256 MB MALL

D_MODEL, D_FF = 4096, 14336
Q5K_BLOCK = 176               # bytes per Q5_K super-block
Q6K_BLOCK = 210               # bytes per Q6_K block
Q3K_BLOCK = 110               # bytes per Q3_K block
SWEEP_M = (1, 2, 4, 8, 16, 32)
LAYERS = 8                    # decode GEMVs per q4k_gemv_layers launch in the bench
W8A8_N = W8A8_K = 3072
W8A8_M = (1024, 8192)


# The source pages' own numbers for this computation, on their hardware: context for the
# reader, not targets (no page reports a Q4_K GB/s or TFLOP/s, so vs_baseline is null).
PAGES_CONTEXT = [
    {"figure": "2.04 -> 2.21 tokens/s decode after the improved Q4_K quant loading",
     "hardware": "Intel Arc GPUs (ESIMD/SYCL)",
     "source": "Writing an ESIMD Fused Kernel From Reverse-Engineered Assembly, Getting Q4_K Right"},
    {"figure": "pp512 1.18x and tg128 1.04x of llama.cpp (gemma-4-12B Q4_K_M)",
     "hardware": "AMD zen2 Threadripper 3990X (CPU)",
     "source": "CPU kernel parity: decode and tile kernels at llama.cpp speed, Validation"},
    {"figure": "INT8 W8A8 linear 15-17% faster than BF16 at M = 1024 (K = N = 3072)",
     "hardware": "Intel Arc B580 (Xe2)",
     "source": "xpu-kernels, Headline result"},
]


def q4k_bytes(n, k):
    return n * (k // 256) * 144


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (used for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget for the oracle baseline")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one device copy of 256 MiB (counter calibration)")
    p.add_argument("--only", default="",
                   help="comma list of kernels to run "
                        "(gemv,layers,q5k_gemv,q6k_gemv,q3k_gemv,sweep_gemv,sweep_gemm,mlp,gemm,q5k_gemm,"
                        "q6k_gemm,q3k_gemm,"
                        "dequant,w8a8,"
                        "read_probe)")
    p.add_argument("--no-check", action="store_true", help="skip the post-run parity spot check")
    p.add_argument("--eager-only", action="store_true",
                   help="time only the eagerly enqueued launches (no HIP graph replay)")
    p.add_argument("--no-dispatch-trace", action="store_true",
                   help="skip the per-dispatch device-duration pass (torch.profiler)")
    p.add_argument("--summarize-profile", nargs="+", metavar="DIR",
                   help="summarize rocprofv3 output directories (kernel trace, then optional "
                        "FETCH_SIZE and WRITE_SIZE counter runs) instead of benchmarking")
    p.add_argument("--profile-command", default="", help="command line recorded in the summary")
    p.add_argument("--out", default="", help="summary output file (markdown)")
    p.add_argument("--workload-hint", default="", help="the --only value the profiled run used")
    return p.parse_args()


def read_probe_runner(_lib, rot, nbytes, torch):
    """Launch the streaming read probe over the first array of each rotating copy: the
    plain-read ceiling that a weight-streaming kernel of the same footprint can reach."""
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def run(i, sp):
        _lib.check(_lib.q4k_read_probe(rot[i][0].data_ptr(), nbytes, sink.data_ptr(), sp))
    return run


class Rotor:
    """R device copies of a set of host arrays; copy i is used at launch i % R."""

    def __init__(self, torch, arrays, bytes_per_set):
        import numpy as np
        self.count = max(1, -(-COLD_BYTES // max(1, bytes_per_set)))
        base = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]
        self.sets = [base]
        for _ in range(self.count - 1):
            self.sets.append([t.clone() for t in base])

    def __getitem__(self, i):
        return self.sets[i % self.count]


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on exactly one GPU; --gpus %d is not supported "
              "(several GPUs would each hold a slice of the weight rows)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_q4_super_block_amd as q4k
    from gemm_q4_super_block_amd import _lib
    import synth

    only = set(filter(None, args.only.split(",")))
    want = lambda name: not only or name in only  # noqa: E731

    torch.cuda.set_device(0)
    q4k.load_library()
    _lib.check(_lib.q4k_init())
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    dev_name = _lib.q4k_device_name()

    kernels = []  # (name, launch(i), algorithmic bytes, flop)

    # ---- decode GEMV 4096 x 4096
    if want("gemv"):
        n = k = D_MODEL
        w = synth.q4k_weights(n, k, seed=0)
        x = synth.normal_f32(k, seed=0)
        nbytes = q4k_bytes(n, k) + 4 * k + 4 * n
        rot = Rotor(torch, [w, x, np.zeros(n, np.float32)], nbytes)

        def run_gemv(i, sp, rot=rot, n=n, k=k):
            wd, xd, yd = rot[i]
            _lib.check(_lib.q4k_gemv(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), 1, n, k, sp))
        kernels.append(("gemv_4096x4096", run_gemv, nbytes, 2 * n * k, rot))

    # ---- several decode GEMVs per launch: LAYERS independent 4096 x 4096 layers (each its
    #      own W, x, y) in one q4k_gemv_layers launch, against the same layers as separate
    #      q4k_gemv launches (eager, and replayed from one graph as graph_us)
    if want("layers"):
        n = k = D_MODEL
        ws = [synth.q4k_weights(n, k, seed=10 + l) for l in range(LAYERS)]
        xs = [synth.normal_f32(k, seed=10 + l) for l in range(LAYERS)]
        ys = [np.zeros(n, np.float32) for _ in range(LAYERS)]
        nbytes = LAYERS * (q4k_bytes(n, k) + 4 * k + 4 * n)
        rot = Rotor(torch, ws + xs + ys, nbytes)

        def run_layers(i, sp, rot=rot, n=n, k=k):
            t = rot[i]
            _lib.check(_lib.q4k_gemv_layers([a.data_ptr() for a in t[:LAYERS]],
                                            [a.data_ptr() for a in t[LAYERS:2 * LAYERS]],
                                            [a.data_ptr() for a in t[2 * LAYERS:]], n, k, sp))

        def run_separate(i, sp, rot=rot, n=n, k=k):
            t = rot[i]
            for l in range(LAYERS):
                _lib.check(_lib.q4k_gemv(t[l].data_ptr(), t[LAYERS + l].data_ptr(),
                                         t[2 * LAYERS + l].data_ptr(), 1, n, k, sp))
        kernels.append(("gemv_layers_%dx4096x4096" % LAYERS, run_layers, nbytes,
                        LAYERS * 2 * n * k, rot))
        kernels.append(("gemv_separate_%dx4096x4096" % LAYERS, run_separate, nbytes,
                        LAYERS * 2 * n * k, rot))

    # ---- decode GEMV on the Q5_K sibling format, 4096 x 4096
    if want("q5k_gemv"):
        n = k = D_MODEL
        w = synth.q5k_weights(n, k, seed=0)
        x = synth.normal_f32(k, seed=0)
        nbytes = n * (k // 256) * Q5K_BLOCK + 4 * k + 4 * n
        rot = Rotor(torch, [w, x, np.zeros(n, np.float32)], nbytes)

        def run_q5(i, sp, rot=rot, n=n, k=k):
            wd, xd, yd = rot[i]
            _lib.check(_lib.q5k_gemv(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), 1, n, k, sp))
        kernels.append(("q5k_gemv_4096x4096", run_q5, nbytes, 2 * n * k, rot))

    # ---- decode GEMV on the Q6_K sibling format, 4096 x 4096
    if want("q6k_gemv"):
        n = k = D_MODEL
        w = synth.q6k_weights(n, k, seed=0)
        x = synth.normal_f32(k, seed=0)
        nbytes = n * (k // 256) * Q6K_BLOCK + 4 * k + 4 * n
        rot = Rotor(torch, [w, x, np.zeros(n, np.float32)], nbytes)

        def run_q6(i, sp, rot=rot, n=n, k=k):
            wd, xd, yd = rot[i]
            _lib.check(_lib.q6k_gemv(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), 1, n, k, sp))
        kernels.append(("q6k_gemv_4096x4096", run_q6, nbytes, 2 * n * k, rot))

    # ---- decode GEMV on the Q3_K sibling format, 4096 x 4096
    if want("q3k_gemv"):
        n = k = D_MODEL
        w = synth.q3k_weights(n, k, seed=0)
        x = synth.normal_f32(k, seed=0)
        nbytes = n * (k // 256) * Q3K_BLOCK + 4 * k + 4 * n
        rot = Rotor(torch, [w, x, np.zeros(n, np.float32)], nbytes)

        def run_q3(i, sp, rot=rot, n=n, k=k):
            wd, xd, yd = rot[i]
            _lib.check(_lib.q3k_gemv(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), 1, n, k, sp))
        kernels.append(("q3k_gemv_4096x4096", run_q3, nbytes, 2 * n * k, rot))

    # ---- small-batch sweep, W 14336 x 4096
    if want("sweep_gemv") or want("sweep_gemm"):
        n, k = D_FF, D_MODEL
        w = synth.q4k_weights(n, k, seed=0)
        for m in SWEEP_M:
            xf = synth.normal_f32((m, k), seed=0)
            if want("sweep_gemv"):
                nbytes = q4k_bytes(n, k) + 4 * m * k + 4 * m * n
                rot = Rotor(torch, [w, xf, np.zeros((m, n), np.float32)], nbytes)

                def run(i, sp, rot=rot, m=m, n=n, k=k):
                    wd, xd, yd = rot[i]
                    _lib.check(_lib.q4k_gemv(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), m, n, k, sp))
                kernels.append(("sweep_gemv_m%d" % m, run, nbytes, 2 * m * n * k, rot))
            if want("sweep_gemm"):
                xb = synth.bf16_bits(xf)
                nbytes = q4k_bytes(n, k) + 2 * m * k + 4 * m * n
                rot = Rotor(torch, [w, xb.view(np.int16), np.zeros((m, n), np.float32)], nbytes)

                def run(i, sp, rot=rot, m=m, n=n, k=k):
                    wd, xd, yd = rot[i]
                    _lib.check(_lib.q4k_gemm(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), m, n, k, sp))
                kernels.append(("sweep_gemm_m%d" % m, run, nbytes, 2 * m * n * k, rot))

    # ---- SwiGLU MLP at one token
    if want("mlp"):
        wg = synth.q4k_weights(D_FF, D_MODEL, seed=0, stream=synth.W_GATE)
        wu = synth.q4k_weights(D_FF, D_MODEL, seed=0, stream=synth.W_UP)
        wdn = synth.q4k_weights(D_MODEL, D_FF, seed=0, stream=synth.W_DOWN)
        x = synth.normal_f32(D_MODEL, seed=0)
        nbytes = 3 * q4k_bytes(D_FF, D_MODEL) + 4 * D_MODEL + 2 * 4 * D_FF + 4 * D_MODEL
        rot = Rotor(torch, [wg, wu, wdn, x, np.zeros(D_FF, np.float32),
                            np.zeros(D_MODEL, np.float32)], nbytes)

        def run_mlp(i, sp, rot=rot):
            g, u, d, xd, hd, od = rot[i]
            _lib.check(_lib.q4k_swiglu_mlp(g.data_ptr(), u.data_ptr(), d.data_ptr(), xd.data_ptr(),
                                           hd.data_ptr(), od.data_ptr(), D_MODEL, D_FF, sp))
        kernels.append(("swiglu_mlp_4096_14336", run_mlp, nbytes, 2 * 3 * D_FF * D_MODEL, rot))

    # ---- prefill GEMM, M = 512
    if want("gemm"):
        m, k = 512, D_MODEL
        xb = synth.normal_bf16((m, k), seed=0)
        for n in (D_MODEL, D_FF):
            w = synth.q4k_weights(n, k, seed=0)
            nbytes = q4k_bytes(n, k) + 2 * m * k + 4 * m * n
            rot = Rotor(torch, [w, xb.view(np.int16), np.zeros((m, n), np.float32)], nbytes)

            def run(i, sp, rot=rot, m=m, n=n, k=k):
                wd, xd, yd = rot[i]
                _lib.check(_lib.q4k_gemm(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), m, n, k, sp))
            kernels.append(("gemm_512x%dx4096" % n, run, nbytes, 2 * m * n * k, rot))

    # ---- prefill GEMM on Q5_K weights, M = 512, N = K = 4096
    if want("q5k_gemm"):
        m, n, k = 512, D_MODEL, D_MODEL
        xb = synth.normal_bf16((m, k), seed=0)
        w = synth.q5k_weights(n, k, seed=0)
        nbytes = n * (k // 256) * Q5K_BLOCK + 2 * m * k + 4 * m * n
        rot = Rotor(torch, [w, xb.view(np.int16), np.zeros((m, n), np.float32)], nbytes)

        def run_q5g(i, sp, rot=rot, m=m, n=n, k=k):
            wd, xd, yd = rot[i]
            _lib.check(_lib.q5k_gemm(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), m, n, k, sp))
        kernels.append(("q5k_gemm_512x4096x4096", run_q5g, nbytes, 2 * m * n * k, rot))

    # ---- prefill GEMM on the Q6_K and Q3_K sibling formats, M = 512, N = K = 4096
    for fmt, gen, blk, fn in (("q6k", synth.q6k_weights, Q6K_BLOCK, _lib.q6k_gemm),
                              ("q3k", synth.q3k_weights, Q3K_BLOCK, _lib.q3k_gemm)):
        if not want(fmt + "_gemm"):
            continue
        m, n, k = 512, D_MODEL, D_MODEL
        xb = synth.normal_bf16((m, k), seed=0)
        w = gen(n, k, seed=0)
        nbytes = n * (k // 256) * blk + 2 * m * k + 4 * m * n
        rot = Rotor(torch, [w, xb.view(np.int16), np.zeros((m, n), np.float32)], nbytes)

        def run_pg(i, sp, rot=rot, m=m, n=n, k=k, fn=fn):
            wd, xd, yd = rot[i]
            _lib.check(fn(wd.data_ptr(), xd.data_ptr(), yd.data_ptr(), m, n, k, sp))
        kernels.append(("%s_gemm_512x4096x4096" % fmt, run_pg, nbytes, 2 * m * n * k, rot))

    # ---- dequant export (bf16) of the 4096 x 4096 matrix
    if want("dequant"):
        n = k = D_MODEL
        w = synth.q4k_weights(n, k, seed=0)
        nbytes = q4k_bytes(n, k) + 2 * n * k
        rot = Rotor(torch, [w, np.zeros((n, k), np.uint16).view(np.int16)], nbytes)

        def run_dq(i, sp, rot=rot, n=n, k=k):
            wd, od = rot[i]
            _lib.check(_lib.q4k_dequantize_bf16(wd.data_ptr(), od.data_ptr(), n, k, sp))
        kernels.append(("dequant_bf16_4096x4096", run_dq, nbytes, 0, rot))

    # ---- INT8 W8A8 linear layer, K = N = 3072: activation row quantizer (bf16 -> int8 +
    #      scales) and the fused GEMM + dequant epilogue (int8 x, w -> bf16 out)
    if want("w8a8"):
        n, k = W8A8_N, W8A8_K
        for m in W8A8_M:
            x, xs, w, ws, b = synth.w8a8_case(m, n, k, seed=0)
            nbytes = m * k + n * k + 4 * m + 8 * n + 2 * m * n
            rot = Rotor(torch, [x, xs, w, ws, b, np.zeros((m, n), np.int16)], nbytes)

            def run_w8(i, sp, rot=rot, m=m, n=n, k=k):
                xd, xsd, wd, wsd, bd, od = rot[i]
                _lib.check(_lib.w8a8_linear(xd.data_ptr(), xsd.data_ptr(), wd.data_ptr(), wsd.data_ptr(),
                                            bd.data_ptr(), od.data_ptr(), m, n, k, sp))
            kernels.append(("w8a8_linear_%dx%dx%d" % (m, n, k), run_w8, nbytes, 2 * m * n * k, rot))
        m = W8A8_M[0]
        xb = synth.normal_bf16((m, k), seed=0)
        nbytes = 2 * m * k + m * k + 4 * m
        rot = Rotor(torch, [xb.view(np.int16), np.zeros((m, k), np.int8), np.zeros(m, np.float32)], nbytes)

        def run_wq(i, sp, rot=rot, m=m, k=k):
            xd, qd, sd = rot[i]
            _lib.check(_lib.w8a8_quantize_rows(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(), m, k, sp))
        kernels.append(("w8a8_quantize_%dx%d" % (m, k), run_wq, nbytes, 0, rot))

    # ---- plain streaming read of the weight footprints (ceilings for the GEMV path: the
    #      decode weight, one 14336 x 4096 matrix, and the gate/up pair)
    if want("read_probe"):
        for n, k in ((D_MODEL, D_MODEL), (D_FF, D_MODEL), (2 * D_FF, D_MODEL)):
            nbytes = q4k_bytes(n, k)
            rot = Rotor(torch, [synth.q4k_weights(n, k, seed=0)], nbytes)
            kernels.append(("read_probe_%d" % nbytes, read_probe_runner(_lib, rot, nbytes, torch),
                            nbytes, 0, rot))
        # 1 GiB, four times the MALL: the rate HBM sustains once launch and ramp costs
        # are amortized (the asymptotic read ceiling)
        nbytes = 1 << 30
        rot = Rotor(torch, [np.full(nbytes, 3, np.uint8)], nbytes)
        kernels.append(("read_probe_%d" % nbytes, read_probe_runner(_lib, rot, nbytes, torch),
                        nbytes, 0, rot))

    if args.copy_probe:
        # one elementwise kernel that reads 256 MiB and writes 256 MiB: the reference
        # dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        print("copy probe: elementwise kernel read and wrote 268435456 bytes", file=sys.stderr)

    torch.cuda.synchronize()
    # warm-up (also sets each kernel's per-device launch attributes)
    for s in range(args.warmup):
        for _, run, *_ in kernels:
            run(s, sp)
    torch.cuda.synchronize()

    # Timed region: each kernel's K launches back to back on the launch stream
    # (torch's current stream), between two HIP events recorded on that stream.
    # The per-launch average (launch gaps included) is the kernel's duration,
    # the figure the roofline fractions use.  Besides it:
    #   * the same K launches captured once into a HIP graph and replayed
    #     (graph_us: what a caller that records its decode step pays);
    #   * per-dispatch device durations (start to end timestamps of every
    #     dispatch, from the runtime's activity trace through torch.profiler,
    #     the same timestamps rocprofv3's kernel trace reads): median, p10 and
    #     p90 over the K launches (dispatch_us).
    ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # noqa: E731
    eager_ev = [ev() for _ in kernels]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (name, run, *_), (e0, e1) in zip(kernels, eager_ev):
        e0.record(stream)
        for s in range(args.steps):
            run(args.warmup + s, sp)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    graph_ms = [None] * len(kernels)
    if not args.eager_only:
        cap = torch.cuda.Stream()
        graph_ev = [ev() for _ in kernels]
        for i, (name, run, *_) in enumerate(kernels):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for s in range(args.steps):
                    run(args.warmup + s, cap.cuda_stream)
            g.replay()  # the first replay uploads the graph
            torch.cuda.synchronize()
            e0, e1 = graph_ev[i]
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            graph_ms[i] = e0.elapsed_time(e1)
            del g
    dispatch = [None] * len(kernels)
    if not args.no_dispatch_trace:
        for i, (name, run, *_) in enumerate(kernels):
            dispatch[i] = dispatch_durations(torch, lambda run=run: [
                run(args.warmup + s, sp) for s in range(args.steps)], args.steps)

    per = {}
    total_ms = 0.0
    for i, (name, run, nbytes, flop, rot) in enumerate(kernels):
        ms = eager_ev[i][0].elapsed_time(eager_ev[i][1])
        total_ms += ms
        us = ms * 1e3 / args.steps
        r = {"us": round(us, 3), "copies": rot.count}
        if graph_ms[i] is not None:
            r["graph_us"] = round(graph_ms[i] * 1e3 / args.steps, 3)
        if dispatch[i]:
            r["dispatch_us"] = dispatch[i]
        if nbytes:
            r["gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            r["hbm_frac"] = round(r["gbs"] / HBM_PEAK_GBS, 4)
        if flop:
            r["tflops"] = round(flop / (us * 1e-6) / 1e12, 2)
        if name.startswith("gemm_") or name.startswith("sweep_gemm") or name.startswith(("q5k_gemm", "q6k_gemm", "q3k_gemm")):
            r["mfma_frac"] = round(r["tflops"] / BF16_PEAK_TFLOPS, 4)
        if name.startswith("w8a8_linear"):
            r["tops"] = r.pop("tflops")
            r["mfma_frac"] = round(r["tops"] / INT8_PEAK_TOPS, 4)
        per[name] = r

    check = None if args.no_check else spot_check(kernels, args, np, torch)

    head = per.get("gemv_4096x4096")
    gemm = per.get("gemm_512x4096x4096")
    mlp = per.get("swiglu_mlp_4096_14336")
    w8 = per.get("w8a8_linear_%dx%dx%d" % (W8A8_M[0], W8A8_N, W8A8_K))
    value = head["gbs"] if head else None
    cpu = None if args.no_cpu_baseline or not head else cpu_baseline(args, np)
    crossover = None
    if all(("sweep_gemv_m%d" % m) in per and ("sweep_gemm_m%d" % m) in per for m in SWEEP_M):
        crossover = next((m for m in SWEEP_M
                          if per["sweep_gemm_m%d" % m]["us"] < per["sweep_gemv_m%d" % m]["us"]), None)

    def timing(r):
        t = {"eager_us": r["us"]}
        if "graph_us" in r:
            t["graph_us"] = r["graph_us"]
        if "dispatch_us" in r:
            t["dispatch_us"] = {key: r["dispatch_us"][key] for key in ("median", "p10", "p90", "n")}
        return t

    out = {
        "metric": "Q4_K GEMV eff. HBM GB/s (% of peak); M=512 GEMM TFLOP/s (% MFMA peak)",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": "the decode GEMV computes in f32 (Q4_K weights, f32 x, f32 FMA and "
                        "accumulation); the prefill GEMM in bf16 MFMA with f32 accumulation",
        "data": "synthetic (seeded; Q4_K fields uniform, d/dmin |N(0,1)|*0.01, activations N(0,1))",
        "config": {
            "workload": "decode GEMV y = W x, W 4096 x 4096 Q4_K (9,437,184 B), x/y fp32, "
                        "cold weights (%d rotating copies)" % (head["copies"] if head else 0),
            "prefill_gemm": "Y = X W^T, X bf16 [512, 4096], W 4096 x 4096 Q4_K",
            "mlp": "SwiGLU 4096 -> 14336 -> 4096 at one token",
            "sweep": "W 14336 x 4096, M in %s" % (list(SWEEP_M),),
            "w8a8": "INT8 W8A8 linear, int8 x [M, 3072] and w [3072, 3072] with fp32 row scales "
                    "and bias -> bf16, M in %s; bf16 row quantizer at M = %d" % (list(W8A8_M), W8A8_M[0]),
        },
        "timing_note": "us / gbs / tflops: the per-launch average of K back-to-back launches "
                       "between HIP events on the launch stream (the roofline figures use it); "
                       "dispatch_us: per-dispatch device durations (median, p10, p90) from the "
                       "runtime's activity trace; graph_us: the same K launches replayed from "
                       "one HIP graph",
        "percent_of_peak": {
            "gemv_hbm": round(100 * head["hbm_frac"], 2) if head else None,
            "gemm_m512_mfma_bf16": round(100 * gemm["mfma_frac"], 2) if gemm else None,
        },
        "gemm_m512_tflops": gemm["tflops"] if gemm else None,
        "read_ceiling_gbs": {name[len("read_probe_"):]: r["gbs"] for name, r in per.items()
                             if name.startswith("read_probe_")} or None,
        "roofline": None,
        "roofline_gemm": None,
        "roofline_mlp": None,
        "roofline_w8a8": None,
        "cpu_baseline": cpu,
        "layers": layers_summary(per),
        "context": PAGES_CONTEXT,
        "kernels": per,
        "sweep_crossover_m": crossover,
        "parity_spot_check": check,
        "device": dev_name,
        "wall_s": round(wall, 3),
    }
    if head:
        out["roofline"] = {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": head["hbm_frac"], "traffic": traffic("gemv_4096x4096"),
                           "kernel": "k_gemv_decode",
                           "bytes_per_launch": 9469952, **timing(head)}
    if gemm:
        out["roofline_gemm"] = {"bound": "mfma", "achieved": gemm["tflops"], "peak": BF16_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": gemm["mfma_frac"],
                                "traffic": traffic("gemm_512x4096x4096"),
                                "kernel": "k_gemm_q4k_kslice<2, 2, 4>",
                                "flop_per_launch": 2 * 512 * 4096 * 4096, **timing(gemm)}
    if mlp:
        out["roofline_mlp"] = {"bound": "hbm", "achieved": mlp["gbs"], "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": mlp["hbm_frac"],
                               "traffic": mlp_traffic(),
                               "kernels": "k_gemv_decode<8, 1, true, 4> (gate/up + SwiGLU), "
                                          "k_gemv_decode<8, 4, false, 4> (down)",
                               "bytes_per_launch": 3 * q4k_bytes(D_FF, D_MODEL) + 4 * D_MODEL
                               + 2 * 4 * D_FF + 4 * D_MODEL, **timing(mlp)}
    if w8:
        out["roofline_w8a8"] = {"bound": "mfma", "achieved": w8["tops"], "peak": INT8_PEAK_TOPS,
                                "unit": "TOP/s", "frac": w8["mfma_frac"],
                                "traffic": traffic("w8a8_linear_%dx%dx%d" % (W8A8_M[0], W8A8_N, W8A8_K)),
                                "kernel": "k_w8a8_gemm<1, 3, 3, 1>",
                                "op_per_launch": 2 * W8A8_M[0] * W8A8_N * W8A8_K, **timing(w8)}
    print(json.dumps(out))


# Sources each workload's kernels are compiled from (a traffic figure is used only while
# the code of its kernels is unchanged since the counters were taken).
_COMMON_SOURCES = ("q4k_device.h", "q4k_launch.h")
KERNEL_SOURCES = {
    "gemv": ("k_gemv.hip", "k_gemv_split.hip"),
    "gemm": ("k_gemm.hip", "k_gemm_stream.hip", "lds_copy.h"),
    "dequant": ("k_dequant.hip",),
    "w8a8": ("k_w8a8.hip", "lds_copy.h"),
    "planes": ("k_planes.hip",),
}


def _family(workload):
    if workload.startswith("w8a8"):
        return "w8a8"
    if workload.startswith("q6k") or workload.startswith("q3k"):
        return "planes"
    if "gemm" in workload:
        return "gemm"
    if workload.startswith("dequant") or workload.startswith("read_probe"):
        return "dequant"
    return "gemv"


def _code_only(text):
    """C++ source without comments and with whitespace runs collapsed: what the compiler
    sees, so that a comment edit does not mark the measured kernels as changed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[_family(workload)] + _COMMON_SOURCES:
        with open(os.path.join(ROOT, "gemm_q4_super_block_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic(name):
    """HBM bytes per launch measured by rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by the
    elementwise-kernel calibration) for workload `name`, from the summaries in profiles/,
    or None if none covers it or the kernel sources changed since it was taken."""
    import glob
    current = kernel_source_hash(name)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        try:
            with open(path) as f:
                for line in f:
                    if line.startswith("traffic_json: "):
                        t = json.loads(line[len("traffic_json: "):])
                        if (t.get("source_hashes", {}).get(name) == current
                                and name in t.get("bytes_per_launch", {})):
                            return t["bytes_per_launch"][name]
        except (OSError, ValueError):
            continue
    return None


def mlp_traffic():
    """The SwiGLU MLP's HBM bytes per call: its two launches' counter figures added, or None."""
    parts = [traffic("swiglu_mlp_gateup_%dx%d" % (D_FF, D_MODEL)),
             traffic("swiglu_mlp_down_%dx%d" % (D_MODEL, D_FF))]
    return None if None in parts else sum(parts)


def _template_args(name, kernel):
    """Template arguments of `kernel<...>` in a demangled name, as a tuple of strings."""
    i = name.find(kernel + "<")
    if i < 0:
        return None
    j = name.index(">", i)
    return tuple(a.strip() for a in name[i + len(kernel) + 1:j].split(","))


# Dispatch signatures of the timed kernels -> workload.  Grid sizes (total work-items) and
# LDS sizes follow from the launch code for these shapes.
def dispatch_workload(name, threads, lds, hint=""):
    if "k_gemv_layers" in name:
        return "gemv_layers_%dx4096x4096" % LAYERS
    dc = _template_args(name, "k_gemv_decode")
    if dc:
        # <NW, NS, GLU, FMT>: 8 rows per workgroup of 64 NW threads, NS K steps of 4096
        ns, glu, fmt = dc[1], dc[2], dc[3]
        rows = threads // 64
        if glu == "true":
            return "swiglu_mlp_gateup_14336x4096"
        if fmt == "5":
            return "q5k_gemv_4096x4096" if rows == 4096 and ns == "1" else "q5k_other"
        if ns == "4" and rows == 4096:
            return "swiglu_mlp_down_4096x14336"
        if ns == "1" and rows == 4096:
            return "gemv_4096x4096"
        if ns == "1" and rows == 14336:
            return "sweep_gemv_14336x4096_m1"
        return "gemv_other"
    gv = _template_args(name, "k_gemv_q4k")
    if gv:
        # <MT, R, GLU, NWV, FMT>
        mt, glu, fmt = gv[0], gv[2], gv[4] if len(gv) > 4 else "4"
        if glu == "true":
            return "swiglu_mlp_gateup_other"
        if fmt == "5":
            return "q5k_other"
        if mt == "1":
            return "gemv_other"
        return "sweep_gemv_14336x4096_batched"
    dq = _template_args(name, "k_dequant_q4k")
    if dq:
        return "dequant_bf16_4096x4096" if dq == ("true", "4") else "dequant_other"
    if _template_args(name, "k_gemm_q4k_stream"):
        return "sweep_gemm_14336x4096"
    if "k_gemm_q4k_128x256" in name:
        return "gemm_512x14336x4096" if threads == 57344 else "gemm_other"
    ks = _template_args(name, "k_gemm_q4k_kslice")
    if ks:
        # <TI, NJ, FMT>: 64 x 128 tiles (TI = 2) at m=512, n=4096; 32 x 64 (TI = 1) for m <= 32
        if ks == ("2", "2", "4"):
            return "gemm_512x4096x4096" if threads == 131072 else "gemm_other"
        if ks == ("2", "2", "5"):
            return "q5k_gemm_512x4096x4096" if threads == 131072 else "q5k_gemm_other"
        if ks == ("1", "2", "4"):
            return "sweep_gemm_14336x4096"
        return "q5k_gemm_other"
    sk = _template_args(name, "k_gemm_q4k")
    if sk and len(sk) > 5 and sk[5] == "5":
        return "q5k_gemm_512x4096x4096"
    if "k_gemm_q4k<4, 1, 1, 4, 2>" in name:
        return "gemm_other"
    if "k_gemm_q4k<1, 4, 1, 1, 2>" in name:
        return "sweep_gemm_14336x4096"
    if "k_read_probe" in name:
        return "read_probe"
    if "k_gemv_split" in name:
        return "sweep_gemv_14336x4096_split"
    gp = _template_args(name, "k_gemv_planes") or _template_args(name, "k_gemv_planes_lds")
    if gp:
        # <FMT, WAVES, RPW, MT>: one wave per RPW weight rows
        rows = threads // 64 * int(gp[2])
        return ("q%sk_gemv_4096x4096" % gp[0]) if rows == 4096 and gp[3] == "1" else "planes_other"
    if "k_dequant_planes" in name:
        return "planes_dequant"
    pl = _template_args(name, "k_gemm_planes_lds")
    if pl:
        # <FMT>: 128 x 128 tiles of 8 waves, split K in two at M = 512 (32 x 4 x 2 workgroups)
        return ("q%sk_gemm_512x4096x4096" % pl[0]) if threads == 32 * 4 * 2 * 512 else "planes_other"
    pg = _template_args(name, "k_gemm_planes")
    if pg:
        # <FMT, WAVES_M, WAVES_N, TI, TJ>: 128 x 128 tiles, split K in two at M = 512
        big = pg[1:] == ("4", "1", "1", "4")
        return ("q%sk_gemm_512x4096x4096" % pg[0]) if big and threads == 128 * 2 * 256 else "planes_other"
    if "k_zero_planes" in name:
        return "split_k_zero_fill"
    wg = _template_args(name, "k_w8a8_gemm")
    if wg:
        # <TI, TJ, S, OUT>: (64 TI) x (64 TJ) tiles of the 3072-wide output, 256 threads each
        # (64 x 192 at M = 1024, 128 x 192 at M = 8192)
        if wg == ("1", "3", "3", "1") and threads == (3072 // 192) * (1024 // 64) * 256:
            return "w8a8_linear_1024x3072x3072"
        if wg == ("2", "3", "2", "1") and threads == (3072 // 192) * (8192 // 128) * 256:
            return "w8a8_linear_8192x3072x3072"
        return "w8a8_other"
    if "k_w8a8_quantize_rows" in name:
        return "w8a8_quantize_1024x3072" if threads == 1024 * 64 else "w8a8_other"
    if "k_zero_f32" in name:
        return "split_k_zero_fill"
    if "copy" in name.lower() or "elementwise" in name:
        return "copy"
    return "other"


def _short_name(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _dirs, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    return None


def summarize_profile(args):
    """Write a markdown summary of rocprofv3 runs: per-workload kernel durations from the
    kernel trace; with counter runs, HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, KiB,
    scaled by what the same counters read for the 256 MiB copy probe), and with a fourth
    directory the MFMA and VALU utilization of each kernel."""
    import statistics
    dirs = args.summarize_profile
    trace = _read_csv(_find(dirs[0], "kernel_trace.csv"))
    groups = {}
    for r in trace:
        name = r["Kernel_Name"]
        key = (_short_name(name), int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]),
               int(r["Grid_Size_Z"]), int(r["LDS_Block_Size"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 kernel summary", "", "Command:", "", "```", args.profile_command or "(not recorded)",
             "```", "", "Kernel durations per dispatch (us), grouped by kernel and launch shape:", "",
             "| workload | kernel | grid (threads) | LDS B | calls | median | mean | p10 | p90 |",
             "|---|---|---|---|---|---|---|---|---|"]
    per_workload = {}
    for key, v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        kname, gx, gy, gz, lds = key
        wl = dispatch_workload(kname, gx * gy * gz, lds, args.workload_hint)
        v.sort()
        med = statistics.median(v)
        per_workload.setdefault(wl, med)
        lines.append("| %s | `%s` | %dx%dx%d | %d | %d | %.3f | %.3f | %.3f | %.3f |" % (
            wl, kname[:60], gx, gy, gz, lds, len(v), med, statistics.fmean(v), v[len(v) // 10],
            v[(9 * len(v)) // 10]))
    traffic_bytes = {}
    if len(dirs) >= 3:
        counters = {}
        for d in dirs[1:3]:
            for r in _read_csv(_find(d, "counter_collection.csv")):
                kname = _short_name(r["Kernel_Name"])
                gx = int(r["Grid_Size"]) if "Grid_Size" in r else 0
                lds = int(r.get("LDS_Block_Size", 0))
                counters.setdefault((kname, r["Counter_Name"], lds, gx), []).append(float(r["Counter_Value"]))
        # calibration: the copy probe moves 256 MiB each way
        cal = {}
        for (kname, cname, lds, gx), vals in counters.items():
            if "elementwise" in kname:
                cal[cname] = max(cal.get(cname, 0.0), max(vals))
        lines += ["", "HBM traffic per dispatch from counters (KiB), median over dispatches:", "",
                  "| kernel | LDS B | grid | FETCH_SIZE | WRITE_SIZE |", "|---|---|---|---|---|"]
        scale = {c: (262144.0 / cal[c] if cal.get(c) else None) for c in ("FETCH_SIZE", "WRITE_SIZE")}
        seen = {}
        for (kname, cname, lds, gx), vals in counters.items():
            seen.setdefault((kname, lds, gx), {})[cname] = statistics.median(vals)
        for (kname, lds, gx), cs in sorted(seen.items()):
            lines.append("| `%s` | %d | %d | %.1f | %.1f |" % (kname[:60], lds, gx, cs.get("FETCH_SIZE", -1),
                                                            cs.get("WRITE_SIZE", -1)))
            wl = dispatch_workload(kname, gx, lds, args.workload_hint)
            if scale["FETCH_SIZE"] and scale["WRITE_SIZE"] and wl not in ("other", "copy"):
                traffic_bytes.setdefault(wl, round((cs.get("FETCH_SIZE", 0) * scale["FETCH_SIZE"] +
                                                    cs.get("WRITE_SIZE", 0) * scale["WRITE_SIZE"]) * 1024))
        lines += ["", "Calibration: an elementwise kernel that reads and writes 256 MiB (262144 KiB each way) "
                  "read FETCH_SIZE = %s KiB and WRITE_SIZE = %s KiB; scale factors (262144 / reading): %s." % (
                      cal.get("FETCH_SIZE"), cal.get("WRITE_SIZE"), scale)]
    if len(dirs) >= 4:
        # Utilization pass: MfmaUtil (% of SIMD cycles with the matrix core busy), VALUBusy (% of
        # CU cycles issuing VALU) and the bf16 MFMA FLOP count (MOPS x 512).
        util = {}
        for r in _read_csv(_find(dirs[3], "counter_collection.csv")):
            kname = _short_name(r["Kernel_Name"])
            gx = int(r["Grid_Size"]) if "Grid_Size" in r else 0
            lds = int(r.get("LDS_Block_Size", 0))
            util.setdefault((kname, lds, gx), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        lines += ["", "Compute utilization per dispatch from counters, median over dispatches "
                  "(MFMA ops = SQ_INSTS_VALU_MFMA_MOPS_BF16 or _I8 x 512):", "",
                  "| kernel | LDS B | grid | MfmaUtil % | VALUBusy % | MFMA ops |", "|---|---|---|---|---|---|"]
        for (kname, lds, gx), cs in sorted(util.items()):
            if "elementwise" in kname or "copyBuffer" in kname:
                continue
            med = {c: statistics.median(v) for c, v in cs.items()}
            mops, kind = med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16"), "bf16"
            if "SQ_INSTS_VALU_MFMA_MOPS_I8" in med:
                mops, kind = med["SQ_INSTS_VALU_MFMA_MOPS_I8"], "int8"
            lines.append("| `%s` | %d | %d | %.1f | %.1f | %s |" % (
                kname[:60], lds, gx, med.get("MfmaUtil", -1), med.get("VALUBusy", -1),
                "%.4g %s" % (mops * 512, kind) if mops else "0"))
    if traffic_bytes:
        lines += ["", "traffic_json: " + json.dumps(
            {"source_hashes": {wl: kernel_source_hash(wl) for wl in traffic_bytes},
             "bytes_per_launch": traffic_bytes})]
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def spot_check(kernels, args, np, torch):
    """Check the last launch of each kernel against the oracle on sampled outputs."""
    import oracle
    import synth
    res = {}
    last = args.warmup + args.steps - 1
    for name, run, nbytes, flop, rot in kernels:
        t = rot[last]
        if name == "gemv_4096x4096":
            w, x, y = (a.cpu().numpy() for a in t)
            rows = np.arange(0, 4096, 37)
            yr, a = oracle.gemv_rows(w, x, 4096, 4096, rows)
            res[name] = float((np.abs(y[rows] - yr[0]) / (1e-4 * a[0])).max())
        elif name.startswith("gemv_layers_"):
            arrs = [a.cpu().numpy() for a in t]
            worst = 0.0
            for l in range(LAYERS):
                w, x, y = arrs[l], arrs[LAYERS + l], arrs[2 * LAYERS + l]
                rows = np.arange(l, 4096, 97)
                yr, a = oracle.gemv_rows(w, x, 4096, 4096, rows)
                worst = max(worst, float((np.abs(y[rows] - yr[0]) / (1e-4 * a[0])).max()))
            res[name] = worst
        elif name == "q5k_gemv_4096x4096":
            w, x, y = (a.cpu().numpy() for a in t)
            rows = np.arange(0, 4096, 37)
            yr, a = oracle.q5k_gemv_rows(w, x, 4096, 4096, rows)
            res[name] = float((np.abs(y[rows] - yr[0]) / (1e-4 * a[0])).max())
        elif name == "q6k_gemv_4096x4096":
            w, x, y = (a.cpu().numpy() for a in t)
            rows = np.arange(0, 4096, 37)
            yr, a = oracle.q6k_gemv_rows(w, x, 4096, 4096, rows)
            res[name] = float((np.abs(y[rows] - yr[0]) / (1e-4 * a[0])).max())
        elif name == "q3k_gemv_4096x4096":
            w, x, y = (a.cpu().numpy() for a in t)
            rows = np.arange(0, 4096, 37)
            yr, a = oracle.q3k_gemv_rows(w, x, 4096, 4096, rows)
            res[name] = float((np.abs(y[rows] - yr[0]) / (1e-4 * a[0])).max())
        elif name == "q5k_gemm_512x4096x4096":
            w, xb, y = (a.cpu().numpy() for a in t)
            cols = np.arange(0, 4096, 256)
            yr, a = oracle.q5k_gemm_cols(w, xb.view(np.uint16), 4096, 4096, cols)
            res[name] = float((np.abs(y[:, cols] - yr) / (1e-2 * a)).max())
        elif name in ("q6k_gemm_512x4096x4096", "q3k_gemm_512x4096x4096"):
            w, xb, y = (a.cpu().numpy() for a in t)
            cols = np.arange(0, 4096, 256)
            x = (xb.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            rows_fn = oracle.q6k_gemv_rows if name.startswith("q6k") else oracle.q3k_gemv_rows
            yr, a = rows_fn(w, x, 4096, 4096, cols)  # bf16 X is exact in fp32
            res[name] = float((np.abs(y[:, cols] - yr) / (1e-2 * a)).max())
        elif name.startswith("gemm_512"):
            w, xb, y = (a.cpu().numpy() for a in t)
            n = y.shape[1]
            cols = np.arange(0, n, n // 16)
            yr, a = oracle.gemm_cols(w, xb.view(np.uint16), n, 4096, cols)
            res[name] = float((np.abs(y[:, cols] - yr) / (1e-2 * a)).max())
        elif name.startswith("w8a8_linear"):
            x, xs, w, ws, b, o = (a.cpu().numpy() for a in t)
            cols = np.arange(0, o.shape[1], 97)
            ref = oracle.w8a8_linear_cols(x, xs, w, ws, b, cols)
            res[name + "_bits_differing"] = int((o.view(np.uint16)[:, cols] != ref).sum())
        elif name.startswith("w8a8_quantize"):
            xb, q, sc = (a.cpu().numpy() for a in t)
            rows = np.arange(0, xb.shape[0], 61)
            rq, rs = oracle.w8a8_quantize_rows(xb.view(np.uint16)[rows])
            res[name + "_bits_differing"] = int((q[rows] != rq).sum() +
                                                (sc[rows].view(np.uint32) != rs.view(np.uint32)).sum())
        elif name == "swiglu_mlp_4096_14336":
            g, u, d, x, h, o = (a.cpu().numpy() for a in t)
            yr, a = oracle.gemv(d.reshape(4096, -1), h, 4096, D_FF)
            res[name + "_down_stage"] = float((np.abs(o - yr[0]) / (1e-4 * a[0])).max())
    return {"max_err_over_tol": res}


def layers_summary(per):
    """The decode GEMVs of LAYERS independent 4096 x 4096 layers: one q4k_gemv_layers launch
    against the same layers launched one by one (eager) and replayed from a graph."""
    one = per.get("gemv_layers_%dx4096x4096" % LAYERS)
    sep = per.get("gemv_separate_%dx4096x4096" % LAYERS)
    if not one or not sep:
        return None
    r = {"layers": LAYERS, "bytes_per_launch": LAYERS * 9469952,
         "one_launch_us": one["us"], "one_launch_gbs": one["gbs"], "one_launch_hbm_frac": one["hbm_frac"],
         "separate_us": sep["us"], "separate_gbs": sep["gbs"],
         "speedup_vs_separate": round(sep["us"] / one["us"], 3)}
    if "graph_us" in sep:
        r["separate_graph_us"] = sep["graph_us"]
        r["speedup_vs_separate_graph"] = round(sep["graph_us"] / one["us"], 3)
    return r


def dispatch_durations(torch, launch_all, launches):
    """Run launch_all() (which enqueues `launches` launches of one bench kernel)
    under torch.profiler and return the per-dispatch device durations in us:
    per HIP kernel name, and per launch (the sum over a launch's kernels, e.g.
    the MLP's gate/up and down), as median / p10 / p90.  None if the trace
    holds no kernel dispatches."""
    import statistics
    from torch.autograd import DeviceType
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        launch_all()
        torch.cuda.synchronize()
    evs = [e for e in prof.profiler.kineto_results.events()
           if e.device_type() == DeviceType.CUDA and not e.name().startswith(("Memcpy", "Memset"))]
    if not evs or len(evs) % launches:
        return None
    evs.sort(key=lambda e: e.start_ns())
    per_launch = len(evs) // launches

    def stats(v):
        v = sorted(v)
        return {"median": round(statistics.median(v), 3), "p10": round(v[len(v) // 10], 3),
                "p90": round(v[(9 * len(v)) // 10], 3), "n": len(v)}
    by_name = {}
    for e in evs:
        by_name.setdefault(_short_name(e.name()), []).append(e.duration_ns() / 1e3)
    launch_sums = [sum(e.duration_ns() for e in evs[j * per_launch:(j + 1) * per_launch]) / 1e3
                   for j in range(launches)]
    out = stats(launch_sums)
    out["kernels_per_launch"] = per_launch
    if per_launch > 1:
        out["by_kernel"] = {k: stats(v) for k, v in by_name.items()}
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, np):
    """The oracle, as it stands, timed on this host's cores on the workloads the GPU runs:
    the decode GEMV (4096 x 4096, every output), the SwiGLU MLP (4096 -> 14336 -> 4096,
    every output) and the M = 512 prefill GEMM (N = K = 4096, a sample of 64 output
    columns, scaled to the full output), each single-threaded (the plain build) and on all
    cores (the OpenMP build: whole output rows per thread, identical results).  Each leg
    repeats whole passes for about cpu_seconds / 6 (at least one pass)."""
    import oracle
    import synth
    budget = max(0.5, args.cpu_seconds / 6.0)
    n = k = D_MODEL
    w = synth.q4k_weights(n, k, seed=0)
    x = synth.normal_f32(k, seed=0)
    wg = synth.q4k_weights(D_FF, D_MODEL, seed=0, stream=synth.W_GATE)
    wu = synth.q4k_weights(D_FF, D_MODEL, seed=0, stream=synth.W_UP)
    wdn = synth.q4k_weights(D_MODEL, D_FF, seed=0, stream=synth.W_DOWN)
    xb = synth.normal_bf16((512, k), seed=0)
    cols = np.arange(0, n, n // 64)
    threads_all = oracle.threads(omp=True)

    def timed(fn):
        fn()  # load and warm the library
        passes, t0 = 0, time.perf_counter()
        while True:
            fn()
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return el / passes, passes

    legs = []
    for omp in (False, True):
        cores = threads_all if omp else 1
        per, p = timed(lambda: oracle.gemv(w, x, n, k, omp=omp))
        legs.append({"workload": "decode_gemv_4096x4096", "cores": cores, "s_per_pass": round(per, 5),
                     "passes": p, "gbs": round((q4k_bytes(n, k) + 4 * k + 4 * n) / per / 1e9, 4),
                     "gflops": round(2 * n * k / per / 1e9, 4)})
        per, p = timed(lambda: oracle.swiglu_mlp(wg, wu, wdn, x, D_MODEL, D_FF, omp=omp))
        mlp_bytes = 3 * q4k_bytes(D_FF, D_MODEL) + 4 * D_MODEL + 2 * 4 * D_FF + 4 * D_MODEL
        legs.append({"workload": "swiglu_mlp_4096_14336", "cores": cores, "s_per_pass": round(per, 5),
                     "passes": p, "gbs": round(mlp_bytes / per / 1e9, 4),
                     "gflops": round(6 * D_FF * D_MODEL / per / 1e9, 4)})
        per, p = timed(lambda: oracle.gemm_cols(w, xb, n, k, cols, omp=omp))
        full = per * n / len(cols)
        legs.append({"workload": "gemm_512x4096x4096", "cores": cores,
                     "s_per_pass": round(per, 5), "passes": p,
                     "sample": "%d of %d output columns" % (len(cols), n),
                     "s_full_output_est": round(full, 4),
                     "tflops": round(2 * 512 * n * k / full / 1e12, 6)})
    head = next(l for l in legs if l["workload"] == "decode_gemv_4096x4096" and l["cores"] == threads_all)
    return {"value": head["gbs"], "unit": "GB/s", "cores": threads_all, "kind": "oracle",
            "sample": "decode GEMV 4096 x 4096 Q4_K, every output, %d passes on %d threads "
                      "(OpenMP over output rows); single-thread and the MLP and GEMM legs in "
                      "'legs'" % (head["passes"], threads_all),
            "host": {"cpu_model": _cpu_model(), "nproc": os.cpu_count(),
                     "affinity_cpus": len(os.sched_getaffinity(0)),
                     "omp_num_threads": os.environ.get("OMP_NUM_THREADS")},
            "legs": legs}


if __name__ == "__main__":
    main()
