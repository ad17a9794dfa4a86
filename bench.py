#!/usr/bin/env python3
"""Benchmark of the QLoRA adapted linear on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  qlora_quantize (fp32 W0 -> NF4 codes + int8/fp32 scales)
  qlora_linear_fwd  y = X.deq(Wq) + (X.A).B
  qlora_linear_bwd  dX, dA, dB (factored; dW never formed)
on the 4096 x 4096 projection, r = 16, M = 2048 tokens, bf16 activations and
adapters.  Inputs are resident in HBM before the timed region; five distinct
W0 buffers (335 MB, more than the 256 MB Infinity Cache) are cycled so every
quantize reads its weights from HBM.

Warm-up runs at least W untimed steps and at least 0.3 s of them (the
chip's clocks ramp over the first tens of milliseconds of load); the steps
actually run are reported as `warmup_steps_run`.

Prints one JSON line.  `value` is fwd+bwd algorithmic TFLOP/s (the dense dW
is not formed and not counted), timed with HIP events around the forward and
backward calls of every timed step; quantize GB/s is reported beside it.
`roofline` covers the dominant kernel (a fused dequantizing GEMM), timed with
HIP events around each of its launches on the stream it runs on, in a second
pass over the same K steps (per-launch events would lengthen the steps that
`value` times).
`cpu_baseline` times the CPU oracle on the same workload (bounded to a few
repetitions of the full step, about 10 s of CPU work).  `decode` reports the
few-token forward (7B-style layer sets, M = 1, 4, 16) in GB/s against HBM.
`uniform4` repeats the timed steps with the uniform 4-bit codebook;
`lora_options` repeats the fwd+bwd steps with the alpha/r factor and dropout
on X.A; `merge`
times folding the adapters into a dense bf16 weight (HBM-bound); `adam`
times one optimizer step of A and B; `loftq_init` times the start of A and B
from the quantization residual.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s & quantize GB/s (% roofline), 4096² r=16"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
N_W0 = 5                      # distinct W0 buffers cycled by the quantize step
SETTLE_S = 0.3                # minimum untimed warm-up time (clock settling)
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="minimum seconds of untimed warm-up steps (clock settling)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time of the oracle baseline")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the few-token (decode) forward measurement")
    p.add_argument("--decode-sets", type=int, default=32,
                   help="distinct 7B layer sets cycled by the decode measurement")
    p.add_argument("--copy-calibrate", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def source_hash():
    h = hashlib.sha256()
    for f in ("gemm.hip", "device.h"):
        with open(os.path.join(ROOT, "quantized_rank_fine_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, launches_flops_key):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if absent or taken on a different kernel source."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_4096x4096_r16_M2048_hbm.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibrate():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


def cpu_baseline(w0, X, dY, A, B, min_seconds):
    """The oracle, as it stands, on the same workload: full quantize of W0
    (fp32 numpy, one thread) and full forward+backward of all tokens
    (dequantize + float64 BLAS matmuls), repeated until `min_seconds` of CPU
    work have been timed (at most 50 repetitions)."""
    import oracle
    from quantized_rank_fine_amd import workloads
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = os.cpu_count()
    n_in, n_out = w0.shape
    M, r = X.shape[0], A.shape[1]
    tq = tf = 0.0
    reps = 0
    while (tq + tf) < min_seconds and reps < 50:
        t0 = time.perf_counter()
        qd = oracle.quantize(w0)
        t1 = time.perf_counter()
        W = oracle.dequantize(qd["packed"], qd["q8"], qd["s2"], n_in, n_out)
        XA, y = oracle.forward(X, W, A, B)
        g = oracle.backward(X, dY, W, A, B, XA)
        t2 = time.perf_counter()
        del W, XA, y, g, qd
        tq += t1 - t0
        tf += t2 - t1
        reps += 1
    flops = workloads.fwd_flops(M, n_in, n_out, r) + workloads.bwd_flops(M, n_in, n_out, r)
    qbytes = workloads.quantize_bytes(n_in, n_out)
    return {
        "value": round(reps * flops / tf / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"the full step {reps} time(s): quantize of the 4096x4096 W0 in fp32 numpy "
                   f"(1 thread, {tq / reps:.2f} s each) and fwd+bwd of all {M} tokens "
                   f"(dequantize + float64 BLAS on {blas} threads, {tf / reps:.2f} s each)"),
        "quantize_GBps": round(reps * qbytes / tq / 1e9, 4),
        "host_cpu_count": os.cpu_count(),
    }


def decode_report(sets, reps=5):
    """Few-token forward of 7B-style layer sets (q, k, v, o 4096x4096; gate,
    up 4096x11008; down 11008x4096), r = 16, M in {1, 4, 16}, bf16.  `sets`
    distinct layer sets (each its own NF4 weights, quantized here from seeded
    N(0, 0.02^2) fp32 weights drawn on the device) are run back to back so the
    weights stream from HBM; the whole sequence is captured once in a HIP
    graph and replayed.  Bytes per linear: codes + int8 block scales + fp32
    group scales + X + A + B + y."""
    import math
    import torch
    from quantized_rank_fine_amd import qlora as q, workloads

    dev = torch.device("cuda:0")
    R = 16
    lins = workloads.LLAMA7B_LINEARS
    g = torch.Generator(device=dev)
    layers = []
    for s in range(sets):
        row = []
        for li, (_, n_in, n_out) in enumerate(lins):
            g.manual_seed(1000003 * s + li)
            w0 = torch.randn(n_in, n_out, device=dev, generator=g) * 0.02
            wq = q.NF4Weight(n_in, n_out, dev)
            q.qlora_quantize(w0, wq)
            del w0
            A = (torch.randn(n_in, R, device=dev, generator=g) / math.sqrt(n_in)).to(torch.bfloat16)
            B = (torch.randn(R, n_out, device=dev, generator=g) * 0.01).to(torch.bfloat16)
            row.append((wq, A, B))
        layers.append(row)
    torch.cuda.synchronize()
    res = {}
    for M in (1, 4, 16):
        g.manual_seed(77 + M)
        X = {n_in: torch.randn(M, n_in, device=dev, generator=g).to(torch.bfloat16)
             for (_, n_in, _) in lins}
        Y = {n_out: torch.empty(M, n_out, dtype=torch.bfloat16, device=dev) for (_, _, n_out) in lins}
        XA = torch.empty(M, R, dtype=torch.float32, device=dev)
        wsb = max(q.qlora_fwd_workspace_bytes(M, n_in, n_out, R) for (_, n_in, n_out) in lins)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

        def seq():
            for s in range(sets):
                for li, (_, n_in, n_out) in enumerate(lins):
                    wq, A, B = layers[s][li]
                    q.qlora_linear_fwd(wq, X[n_in], M, q.BF16, A, B, R, q.BF16, Y[n_out], XA, ws, wsb)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            seq()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            seq()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = sets * sum(workloads.nf4_bytes(n_in, n_out) + M * n_in * 2 + (n_in * R + R * n_out) * 2
                            + M * n_out * 2 for (_, n_in, n_out) in lins)
        gbps = nbytes / (us * 1e-6) / 1e9
        del graph

        # The same sets with the projections that share an input grouped
        # into one qlora_linear_fwd_group call each: q, k, v; o; gate, up;
        # down (four launch pairs per set instead of seven).
        names = [nm for (nm, _, _) in lins]
        groups = [["q", "k", "v"], ["o"], ["gate", "up"], ["down"]]
        Yg = {nm: torch.empty(M, o, dtype=torch.bfloat16, device=dev) for (nm, _, o) in lins}
        XAg = {nm: torch.empty(M, R, dtype=torch.float32, device=dev) for nm in names}
        gws = max(q.qlora_fwd_group_workspace_bytes(M, [lins[names.index(nm)][1] for nm in grp],
                                                    [lins[names.index(nm)][2] for nm in grp], R)
                  for grp in groups)
        wsg = torch.empty(gws, dtype=torch.uint8, device=dev)

        def grouped():
            for s in range(sets):
                for grp in groups:
                    idx = [names.index(nm) for nm in grp]
                    q.qlora_linear_fwd_group([layers[s][i][0] for i in idx],
                                             [X[lins[i][1]] for i in idx], M, q.BF16,
                                             [layers[s][i][1] for i in idx],
                                             [layers[s][i][2] for i in idx], R, q.BF16,
                                             [Yg[nm] for nm in grp], [XAg[nm] for nm in grp],
                                             wsg, gws)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            grouped()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            grouped()
        graph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        usg = e0.elapsed_time(e1) * 1e3 / reps
        gbpsg = nbytes / (usg * 1e-6) / 1e9
        del graph
        res[f"M{M}"] = {"us_per_layer_set": round(us / sets, 2), "GBps": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                        "grouped": {"us_per_layer_set": round(usg / sets, 2),
                                    "GBps": round(gbpsg, 1),
                                    "frac_hbm_peak": round(gbpsg / PEAK_HBM_GBPS, 4)}}
    return {"workload": "7b-layer-decode-r16-bf16", "layer_sets": sets,
            "bytes_per_set_M1": sum(workloads.nf4_bytes(i, o) + i * 2 + (i * R + R * o) * 2 + o * 2
                                    for (_, i, o) in lins),
            "timing": "HIP graph of the whole sequence, replayed; grouped: q/k/v and gate/up "
                      "each one qlora_linear_fwd_group call", **res}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibrate:
        copy_calibrate()
        return

    import numpy as np
    import torch

    from quantized_rank_fine_amd import qlora as q
    from quantized_rank_fine_amd import synth, workloads

    wl = workloads.WORKLOADS[1]
    _, n_in, n_out = wl["linears"][0]
    r, M = wl["rank"], wl["tokens"][0]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16_dev(t):
        return torch.from_numpy(t.raw.view(np.int16)).to(dev).view(torch.bfloat16)

    w0_host = [synth.weights(n_in, n_out, 1, layer=i) for i in range(N_W0)]
    W0s = [torch.from_numpy(w).to(dev) for w in w0_host]
    Xs = synth.activations(M, n_in, 1, "bf16")
    dYs = synth.activations(M, n_out, 1, "bf16", tensor=synth.T_DY)
    As, Bs = synth.adapters(n_in, n_out, r, 1, "bf16")
    X, dY, A, B = bf16_dev(Xs), bf16_dev(dYs), bf16_dev(As), bf16_dev(Bs)
    wq = q.NF4Weight(n_in, n_out, dev)
    Y = torch.empty(M, n_out, dtype=torch.bfloat16, device=dev)
    XA = torch.empty(M, r, dtype=torch.float32, device=dev)
    dX = torch.empty(M, n_in, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(n_in, r, dtype=torch.float32, device=dev)
    dB = torch.empty(r, n_out, dtype=torch.float32, device=dev)
    fwb = q.qlora_fwd_workspace_bytes(M, n_in, n_out, r, q.BF16)
    bwb = q.qlora_bwd_workspace_bytes(M, n_in, n_out, r, q.BF16)
    wsf = torch.empty(fwb, dtype=torch.uint8, device=dev)
    wsb = torch.empty(bwb, dtype=torch.uint8, device=dev)

    def quantize(i):
        q.qlora_quantize(W0s[i % N_W0], wq)

    def fwd_bwd():
        q.qlora_linear_fwd(wq, X, M, q.BF16, A, B, r, q.BF16, Y, XA, wsf, fwb)
        q.qlora_linear_bwd(wq, X, dY, M, q.BF16, A, B, r, q.BF16, XA, dX, dA, dB, wsb, bwb)

    # Untimed warm-up: at least W steps and at least --settle seconds of them,
    # so the timed steps run at the clocks the chip holds under this load (a
    # cold start ramps over the first tens of milliseconds).
    t_w = time.perf_counter()
    n_warm = 0
    while n_warm < args.warmup or time.perf_counter() - t_w < args.settle:
        quantize(n_warm)
        fwd_bwd()
        n_warm += 1
        if n_warm % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        quantize(i)
        ev[i][1].record()
        fwd_bwd()
        ev[i][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # Per-launch kernel times for the roofline: the same K steps once more,
    # with the library's HIP events around each launch of the timed kernels
    # (kept out of the loop above, whose step time they would lengthen).
    q.qlora_timing_reset()
    q.qlora_timing_enable(["quantize", "fwd_gemm", "dx_gemm"])
    for i in range(K):
        quantize(i)
        fwd_bwd()
    torch.cuda.synchronize()
    q.qlora_timing_disable()

    # The uniform 4-bit codebook on the same kernels: the same K steps with a
    # weight quantized to that grid (quantize GB/s and fwd+bwd TFLOP/s).
    wq_u = q.NF4Weight(n_in, n_out, dev, q.CB_UNIFORM4)
    for i in range(args.warmup):
        q.qlora_quantize(W0s[i % N_W0], wq_u)
    evu = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for i in range(K):
        evu[i][0].record()
        q.qlora_quantize(W0s[i % N_W0], wq_u)
        evu[i][1].record()
        q.qlora_linear_fwd(wq_u, X, M, q.BF16, A, B, r, q.BF16, Y, XA, wsf, fwb)
        q.qlora_linear_bwd(wq_u, X, dY, M, q.BF16, A, B, r, q.BF16, XA, dX, dA, dB, wsb, bwb)
        evu[i][2].record()
    torch.cuda.synchronize()

    # The adapter options (alpha/r = 2, dropout p = 0.05 on X.A with a fixed
    # seeded keep mask): the same K fwd+bwd steps through the options entry
    # points.
    keep = (torch.rand(M, r, generator=torch.Generator(device="cpu").manual_seed(11)) >= 0.05)
    keep = keep.to(torch.uint8).to(dev)
    lopt = (2.0, 0.05, keep)
    for _ in range(args.warmup):
        q.qlora_linear_fwd_lora(wq, X, M, q.BF16, A, B, r, q.BF16, *lopt, Y, XA, wsf, fwb)
        q.qlora_linear_bwd_lora(wq, X, dY, M, q.BF16, A, B, r, q.BF16, *lopt, XA, dX, dA, dB,
                                wsb, bwb)
    el0, el1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    el0.record()
    for i in range(K):
        q.qlora_linear_fwd_lora(wq, X, M, q.BF16, A, B, r, q.BF16, *lopt, Y, XA, wsf, fwb)
        q.qlora_linear_bwd_lora(wq, X, dY, M, q.BF16, A, B, r, q.BF16, *lopt, XA, dX, dA, dB,
                                wsb, bwb)
    el1.record()
    torch.cuda.synchronize()
    lora_ms = el0.elapsed_time(el1) / K

    # Merge (fold the adapters into a dense bf16 weight), K launches.
    Wm = torch.empty(n_in, n_out, dtype=torch.bfloat16, device=dev)
    q.qlora_merge(wq, A, B, r, q.BF16, Wm, q.BF16)
    em0, em1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    em0.record()
    for i in range(K):
        q.qlora_merge(wq, A, B, r, q.BF16, Wm, q.BF16)
    em1.record()
    torch.cuda.synchronize()
    merge_us = em0.elapsed_time(em1) * 1e3 / K
    nw = n_in * n_out
    merge_bytes = nw // 2 + nw // 64 + 4 * ((nw // 64 + 255) // 256) + 2 * r * (n_in + n_out) + 2 * nw
    merge = {"us": round(merge_us, 2), "algorithmic_bytes": merge_bytes,
             "GBps": round(merge_bytes / (merge_us * 1e-6) / 1e9, 1),
             "frac_hbm_peak": round(merge_bytes / (merge_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
             "what": "W = deq(Wq) + A.B written as dense bf16, r = 16"}
    # The same from fp32 adapters (the optimizer's master copies).
    A32, B32 = A.float().contiguous(), B.float().contiguous()
    q.qlora_merge(wq, A32, B32, r, q.F32, Wm, q.BF16)
    torch.cuda.synchronize()
    em0.record()
    for i in range(K):
        q.qlora_merge(wq, A32, B32, r, q.F32, Wm, q.BF16)
    em1.record()
    torch.cuda.synchronize()
    m32_us = em0.elapsed_time(em1) * 1e3 / K
    m32_bytes = merge_bytes + 2 * r * (n_in + n_out)
    merge["fp32_adapters"] = {"us": round(m32_us, 2), "algorithmic_bytes": m32_bytes,
                              "GBps": round(m32_bytes / (m32_us * 1e-6) / 1e9, 1)}
    del Wm, A32, B32

    # Adam step of both adapter matrices (fp32 master copies, bf16 copies for
    # the forward), K times.
    na, nb = n_in * r, r * n_out
    opt = {nm: [torch.zeros(nn, dtype=torch.float32, device=dev) for _ in range(4)]
           for nm, nn in (("A", na), ("B", nb))}
    for nm, (th, gr, _, _) in opt.items():
        th.normal_(0.0, 0.02)
        gr.normal_(0.0, 1e-3)
    a16 = torch.empty(na, dtype=torch.bfloat16, device=dev)
    b16 = torch.empty(nb, dtype=torch.bfloat16, device=dev)
    # The K steps are captured in one HIP graph and replayed, so the time is
    # the kernels' and not the Python launch path's (2 x 3.9 MB per step).
    sgr = torch.cuda.Stream()
    sgr.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sgr):
        q.qlora_adam_step(*opt["A"], 1, 1e-3, theta_bf16=a16)        # warm (uncaptured)
        q.qlora_adam_step(*opt["B"], 1, 1e-3, theta_bf16=b16)
    torch.cuda.current_stream().wait_stream(sgr)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(K):
            q.qlora_adam_step(*opt["A"], i + 1, 1e-3, theta_bf16=a16)
            q.qlora_adam_step(*opt["B"], i + 1, 1e-3, theta_bf16=b16)
    ea0, ea1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea0.record()
    graph.replay()
    ea1.record()
    torch.cuda.synchronize()
    adam_us = ea0.elapsed_time(ea1) * 1e3 / K
    del graph
    # The same Adam step fused into the backward's last launch, against the
    # backward followed by the two Adam launches (K steps each, eager).
    stA = [opt["A"][0], opt["A"][2], opt["A"][3], a16]
    stB = [opt["B"][0], opt["B"][2], opt["B"][3], b16]
    def bwd_then_adam(i):
        q.qlora_linear_bwd(wq, X, dY, M, q.BF16, A, B, r, q.BF16, XA, dX, dA, dB, wsb, bwb)
        q.qlora_adam_step(stA[0], dA.view(-1), stA[1], stA[2], i + 1, 1e-3, theta_bf16=a16)
        q.qlora_adam_step(stB[0], dB.view(-1), stB[1], stB[2], i + 1, 1e-3, theta_bf16=b16)
    def bwd_adam(i):
        q.qlora_linear_bwd_adam(wq, X, dY, M, q.BF16, A, B, r, q.BF16, XA, dX, stA, stB, i + 1,
                                1e-3, wsb, bwb)
    adam_fused = {}
    for name, fn in (("bwd_then_adam_us", bwd_then_adam), ("bwd_adam_fused_us", bwd_adam)):
        for i in range(3):
            fn(i)
        eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        eb0.record()
        for i in range(K):
            fn(i)
        eb1.record()
        torch.cuda.synchronize()
        adam_fused[name] = round(eb0.elapsed_time(eb1) * 1e3 / K, 2)
    adam_bytes = (na + nb) * (16 + 12 + 2)
    adam = {"us_per_step": round(adam_us, 2), "params": na + nb, "algorithmic_bytes": adam_bytes,
            "GBps": round(adam_bytes / (adam_us * 1e-6) / 1e9, 1),
            "what": "Adam step of A and B (fp32, two launches, bf16 copies written; HIP graph)",
            "fused_into_backward": adam_fused}
    del opt

    # LoftQ-style start of A and B (rank 16, 24 probe columns, 2 power
    # iterations): a synchronous call, timed on the host clock.
    kq = 24
    gq = torch.Generator(device="cpu").manual_seed(7)
    omega = torch.randn(n_out, kq, generator=gq).to(dev)
    Aq = torch.empty(n_in, r, dtype=torch.bfloat16, device=dev)
    Bq = torch.empty(r, n_out, dtype=torch.bfloat16, device=dev)
    wsq_b = q.qlora_loftq_workspace_bytes(n_in, n_out, kq)
    wsq = torch.empty(wsq_b, dtype=torch.uint8, device=dev)
    q.qlora_quantize(W0s[0], wq)
    q.qlora_loftq_init(W0s[0], wq, omega, kq, r, 2, Aq, Bq, q.BF16, wsq, wsq_b)
    torch.cuda.synchronize()
    tq0 = time.perf_counter()
    for _ in range(3):
        q.qlora_loftq_init(W0s[0], wq, omega, kq, r, 2, Aq, Bq, q.BF16, wsq, wsq_b)
    loftq = {"ms": round((time.perf_counter() - tq0) * 1e3 / 3, 2), "rank": r, "probe_columns": kq,
             "power_iterations": 2,
             "what": "A, B from a rank-16 SVD of W0 - deq(Wq) (6 GPU residual products + host k x k work)"}
    del wsq

    ms_per_step = (t1 - t0) * 1e3 / K
    q_ms = sum(e[0].elapsed_time(e[1]) for e in ev)
    fb_ms = sum(e[1].elapsed_time(e[2]) for e in ev)
    flops = workloads.fwd_flops(M, n_in, n_out, r) + workloads.bwd_flops(M, n_in, n_out, r)
    qbytes = workloads.quantize_bytes(n_in, n_out)
    value = K * flops / (fb_ms * 1e-3) / 1e12
    q_gbps = K * qbytes / (q_ms * 1e-3) / 1e9
    uq_ms = sum(e[0].elapsed_time(e[1]) for e in evu)
    ufb_ms = sum(e[1].elapsed_time(e[2]) for e in evu)
    uniform4 = {"codebook": "uniform 4-bit grid (16 evenly spaced levels in [-1, 1])",
                "fwd_bwd_TFLOPs": round(K * flops / (ufb_ms * 1e-3) / 1e12, 2),
                "quantize_GBps": round(K * qbytes / (uq_ms * 1e-3) / 1e9, 1),
                "fwd_bwd_ms_per_step": round(ufb_ms / K, 4),
                "quantize_ms_per_step": round(uq_ms / K, 4)}

    lora = {"what": "fwd+bwd with alpha/r = 2 and dropout p = 0.05 on X.A (keep mask given)",
            "fwd_bwd_TFLOPs": round(flops / (lora_ms * 1e-3) / 1e12, 2),
            "fwd_bwd_ms_per_step": round(lora_ms, 4)}

    kernels = {}
    # at this workload the dX GEMM also forms dB = XA^T dY (2 M r out flops)
    per_launch_flops = {"fwd_gemm": 2 * M * n_out * (n_in + r),
                        "dx_gemm": 2 * M * n_in * (n_out + r) + 2 * M * r * n_out}
    for name in ("fwd_gemm", "dx_gemm"):
        tot, n = q.qlora_timing_read(q.KERNELS.index(name))
        avg = tot / max(n, 1)
        ach = per_launch_flops[name] / (avg * 1e-3) / 1e12
        kernels[name] = {"launches": n, "avg_us": round(avg * 1e3, 2),
                         "algorithmic_flop": per_launch_flops[name],
                         "TFLOPs": round(ach, 2), "frac_bf16_peak": round(ach / PEAK_BF16_TFLOPS, 4)}
    tot, n = q.qlora_timing_read(q.KERNELS.index("quantize"))
    qavg = tot / max(n, 1)
    kernels["quantize"] = {"launches": n, "avg_us": round(qavg * 1e3, 2),
                           "algorithmic_bytes": qbytes,
                           "GBps": round(qbytes / (qavg * 1e-3) / 1e9, 1),
                           "frac_hbm_peak": round(qbytes / (qavg * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    dom = max(("fwd_gemm", "dx_gemm"), key=lambda k: kernels[k]["avg_us"])
    roof = {"bound": "mfma", "kernel": dom,
            "achieved": kernels[dom]["TFLOPs"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": kernels[dom]["frac_bf16_peak"],
            "traffic": read_traffic(dom, "flops")}

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02^2) weights, N(0,1) bf16 activations)",
        "config": {"workload": wl["name"], "in": n_in, "out": n_out, "rank": r, "tokens": M,
                   "step": "quantize+fwd+bwd", "w0_buffers_cycled": N_W0},
        "quantize_GBps": round(q_gbps, 2),
        "quantize_frac_hbm": round(q_gbps / PEAK_HBM_GBPS, 4),
        "fwd_bwd_ms_per_step": round(fb_ms / K, 4),
        "quantize_ms_per_step": round(q_ms / K, 4),
        "fwd_bwd_frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "kernels": kernels,
        "uniform4": uniform4,
        "lora_options": lora,
        "merge": merge,
        "adam": adam,
        "loftq_init": loftq,
    }
    if not args.no_decode:
        out["decode"] = decode_report(args.decode_sets)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w0_host[0], Xs.values, dYs.values, As.values,
                                           Bs.values, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
