#!/usr/bin/env python3
"""Benchmark of the W4A4 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gateup70b]
                    [--act-quant dynamic|tensor|channel] [--path two|single]

A step is one pass of the whole hot path over one batch: w4a4_linear =
fused activation transform + per-token INT4 quantization + packing, then the
INT4 x INT4 GEMM with int32 accumulation and the fp16 dequant epilogue.
Inputs are seeded synthetic LLaMA-shaped tensors (workloads/), resident in
HBM before the timed region; weights are merged (P^-1 folded in), quantized
and packed on the GPU beforehand, as a deployment would do offline.

With --act-quant tensor|channel the activation steps are static (fixed
offline from a seeded calibration batch, FPTQuant / MergeQuant): one step
for the tensor, or one per channel migrated into the weights before packing;
the step runs w4a4_linear_static instead.

With --bits 3 the layer runs with 3-bit codes (W3A3, FRM-PTQ page) through
w4a4_linear_bits; the codes stay one per nibble, so the bytes are the same.

With --path single (decode, M <= 16) the step is one w4a4_linear_decode
launch (transform, quantization and GEMM in one kernel) and the roofline
kernel is that kernel, priced at the layer's algorithmic bytes.

With --workload attn8b|attn70b the step is one decode step of attention over
the INT4 KV cache with per-head transforms: w4a4_kv_append of the batch's new
tokens, then w4a4_attn_decode over the ragged contexts (up to 8192 cached
tokens).  Its roofline unit is the w4a4_attn_decode call (query transform,
chunked partial attention, merge) priced at the cache bytes it must read.

With --workload tern_down70b_m{1,8,64}|tern_gateup70b_m{1,8,64} the step is
one w4a4_ternary_gemm call: the ternary-weight (W1.58A16, PT2-LLM page) decode
product Y = X · (alpha T + mu)^T with fp16 activations, weights ternarized on
the GPU beforehand (ITF, 2-bit codes and one (alpha, mu) word per row and
block of 128).  Its roofline unit is that call, priced at the packed weight
bytes plus the activations and outputs.

Prints ONE JSON line.  `value` is TOPS of the whole layer (2*M*N*K integer
ops per step / step time).  `roofline` reports the dominant kernel (the GEMM)
against the INT8 MFMA peak (prefill) or HBM bandwidth (decode), its duration
measured with HIP events on the launch stream.  `cpu_baseline` times the CPU
oracle on the same workload (host cores, float64 numpy).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 linear TOPS + µs/layer; % of INT8 MFMA peak (prefill) / HBM BW (decode)"
PEAK_INT8_TOPS = 5000.0          # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, GB/s
PEAK_FP6_TOPS = 10100.0          # MI355X dense fp6 MFMA, TOP/s
MALL_BYTES = 256 << 20           # Infinity Cache: rotate weight copies past it


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gateup70b",
                    help="linear: qkv8b gateup8b down8b gateup70b down70b_m{1,8,64}; "
                         "attention over the INT4 KV cache: attn8b attn70b; ternary-weight "
                         "decode: tern_down70b_m{1,8,64} tern_gateup70b_m{1,8,64}")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path", choices=["two", "single"], default="two",
                    help="'two' = w4a4_linear (transform kernel, then GEMM kernel; the faster "
                         "path measured on MI355X); 'single' = w4a4_linear_decode (one launch, "
                         "M <= 16 tokens)")
    ap.add_argument("--bits", type=int, choices=[3, 4], default=4,
                    help="code width of weights and activations (3: W3A3, FRM-PTQ)")
    ap.add_argument("--gemm", choices=["int8", "f6"], default="int8",
                    help="matrix pipe of the INT4 x INT4 product: int8 MFMA on unpacked nibbles, or "
                         "fp6 MFMA on codes held exactly as E2M3 (w4a4_linear_f6)")
    ap.add_argument("--act-quant", choices=["dynamic", "tensor", "channel"], default="dynamic",
                    help="activation quantizer: per-token dynamic scales, or static steps "
                         "(one per tensor, or one per channel migrated into the weights)")
    ap.add_argument("--read-ceiling", type=float, default=0.0, metavar="MB",
                    help="only time a plain device read (a sum) of MB megabytes, rotated over "
                         "enough buffers to exceed the 256 MB Infinity Cache: the HBM read "
                         "rate one launch of that size reaches")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain copy of a known number of bytes, for calibrating the HBM
    traffic counters: it must read and write exactly `mib` MiB per launch."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def read_ceiling(mb, steps, warmup):
    """HIP-event timing of a plain read of `mb` MB per launch (the library's
    w4a4_read_probe), the buffers rotated like the benchmark's weight copies;
    the launches go to torch's current stream, where the events are."""
    import torch
    import w4a4_post_quantized_amd as L
    n = int(mb * 1e6) // 16 * 4
    copies = max(3, math.ceil(MALL_BYTES / (4 * n)) + 1)
    bufs = [torch.full((n,), i + 1, dtype=torch.int32, device="cuda:0") for i in range(copies)]
    out = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    for i in range(warmup):
        L.read_probe(bufs[i % copies], out, stream=st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        L.read_probe(bufs[i % copies], out, stream=st)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"read_ceiling_bytes_per_launch": 4 * n, "buffers_rotated": copies,
                      "us_per_launch": round(us, 2), "GBps": round(4 * n / us / 1e3, 1),
                      "fraction_of_8TBps": round(4 * n / us / 1e3 / 8000.0, 4),
                      "steps": steps}), flush=True)


def gemm_bytes(wl, M):
    G = wl.K // wl.group_size
    b = M * wl.K // 2 + 4 * M + wl.N * wl.K // 2 + 2 * wl.N * G + 2 * M * wl.N
    if wl.asymmetric:
        b += 2 * wl.N * G
    return b


def layer_bytes(wl, M):
    """Algorithmic HBM bytes of the whole layer in one kernel: the GEMM's
    operands and output plus the fp16 activations and the fp32 factors (the
    packed activations stay in the workspace, written and read once)."""
    return gemm_bytes(wl, M) + 2 * M * wl.K + 4 * (wl.n1 * wl.n1 + wl.n2 * wl.n2)


def traffic_from_profiles(kernel_tag, workload, source="gemm.hip"):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, "w4a4_post_quantized_amd", "csrc", rec.get("source", source))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


CAL_TOKENS = 256                 # calibration batch for static steps
CAL_SEED_OFFSET = 7919


def calibration_batch(wl, inp):
    import workloads as WL
    return WL.make_calibration_activations(wl, CAL_TOKENS, inp["outlier_channels"],
                                           seed=wl.seed + CAL_SEED_OFFSET)


def cpu_threads():
    """(cores this process may run on, threads numpy's BLAS uses)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas = cores
    return cores, blas


CPU_CHUNK = 512                  # output channels per timed chunk of the oracle's GEMM


def cpu_baseline(wl, inp, budget_s, act_quant="dynamic", bits=4):
    """The CPU oracle on a bounded sample of the same workload.

    Timed: the oracle's activation path (transform, quantize, pack: O1-O4) on
    every token once, and its exact integer GEMM + epilogue (O6-O7) on chunks
    of CPU_CHUNK output channels until `budget_s` seconds of GEMM time,
    projected to all N channels.  Each chunk's weights are merged and
    quantized untimed, as both sides prepare weights offline."""
    import oracle as O
    cores, blas = cpu_threads()
    static = act_quant != "dynamic"
    pc = act_quant == "channel"
    steps = None
    if static:
        Zc = O.kron_transform(calibration_batch(wl, inp), inp["P1"], inp["P2"], inp["c"])
        steps = O.calibrate_steps(Zc, pc).astype(np.float64)
        del Zc
    t0 = time.perf_counter()
    if static:
        act = O.transform_quant_static(inp["X"], inp["P1"], inp["P2"], steps, pc, c=inp["c"])
    else:
        act = O.transform_quant(inp["X"], inp["P1"], inp["P2"], inp["c"], bits=bits)
    ta = time.perf_counter() - t0
    t_gemm, cols = 0.0, 0
    for c0 in range(0, wl.N, CPU_CHUNK):
        rows = slice(c0, min(wl.N, c0 + CPU_CHUNK))
        Wt = O.merge_weights(inp["W"][rows], inp["P1"], inp["P2"], inp["c"])
        if pc:
            Wt = O.migrate_steps(Wt, steps)
        wq = O.quantize_weights(Wt, wl.group_size, wl.asymmetric, bits=bits)
        t1 = time.perf_counter()
        D = O.int_gemm(act["q"], wq["codes"], wq["z"], wq["group_size"])
        O.epilogue(D, act["s_x"], wq["s"])
        t_gemm += time.perf_counter() - t1
        cols += rows.stop - rows.start
        del D, Wt, wq
        if t_gemm >= budget_s:
            break
    tg = t_gemm * wl.N / cols
    t = ta + tg
    ops = 2.0 * wl.M * wl.N * wl.K
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": int(blas), "kind": "oracle",
            "affinity_cores": int(cores), "blas_threads": int(blas), "cpu": cpu_model(),
            "sample": f"{wl.name} ({wl.M}x{wl.K}->{wl.N}): the activation path on all {wl.M} "
                      f"tokens ({ta:.1f} s) and the exact GEMM + epilogue on {cols} of {wl.N} "
                      f"output channels ({t_gemm:.1f} s), projected to all channels; weights "
                      f"prepared untimed",
            "us_per_layer": t * 1e6, "transform_quant_us": ta * 1e6, "gemm_epilogue_us": tg * 1e6}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def event_stats(launch, n):
    """Per-launch durations (HIP events around each launch on the launch
    stream): median, p10 and p90 in microseconds."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record()
        launch(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return {"median": round(float(np.median(d)), 2), "p10": round(float(np.percentile(d, 10)), 2),
            "p90": round(float(np.percentile(d, 90)), 2), "launches": n}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the data-parallel W4A4 linear needs no exchange "
              "between GPUs, so N > 1 is not run here (each GPU would run the same kernel "
              "on its share of tokens).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.read_ceiling:
        read_ceiling(args.read_ceiling, args.steps, args.warmup)
        return
    if args.bits != 4 and (args.act_quant != "dynamic" or args.path != "two"):
        raise SystemExit("--bits 3 runs the dynamic two-launch layer only")
    if args.gemm == "f6" and (args.bits != 4 or args.act_quant != "dynamic" or args.path != "two"):
        raise SystemExit("--gemm f6 runs the dynamic two-launch 4-bit layer only")

    import torch
    import workloads as WL
    import w4a4_post_quantized_amd as L
    from workloads import kv as WKV

    if args.workload in WKV.KV_WORKLOADS:
        attn_main(args)
        return
    from workloads import ternary as WT
    if args.workload in WT.TERN_WORKLOADS:
        tern_main(args)
        return

    wl = WL.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = WL.make_inputs(wl)
    M, K, N = wl.M, wl.K, wl.N

    X = torch.from_numpy(inp["X"]).to(dev)
    P1 = torch.from_numpy(inp["P1"]).to(dev)
    P2 = torch.from_numpy(inp["P2"]).to(dev)

    # offline: merge P^-1 into the weights and quantize, on the GPU
    # weight sets smaller than the Infinity Cache are rotated over enough
    # distinct copies (at least 3) that no call finds its weights cached
    wbytes = N * K // 2
    decode = M <= 64
    copies = 1
    if wbytes < MALL_BYTES:
        copies = max(3, -(-MALL_BYTES // wbytes) + 1)
    Wraw = torch.from_numpy(inp["W"]).to(dev)
    Wt = L.merge_weights(Wraw, P1, P2)
    del Wraw
    static = args.act_quant != "dynamic"
    pc = args.act_quant == "channel"
    steps = None
    if static:
        # offline calibration: range of the transformed calibration batch / 7
        Zc = L.transform(torch.from_numpy(calibration_batch(wl, inp)).to(dev), P1, P2)
        amax = Zc.abs().amax(dim=0) if pc else Zc.abs().amax().reshape(1)
        steps = torch.where(amax > 0, amax / 7.0, torch.ones_like(amax)).contiguous()
        del Zc, amax
        if pc:
            Wt = L.migrate_steps(Wt, steps)
    packs = []
    for i in range(copies):
        packs.append(L.pack_weights_bits(Wt if i == 0 else Wt * (1.0 + 1e-3 * i), wl.group_size,
                                         wl.asymmetric, args.bits))
    del Wt
    desc = packs[0][0]
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.empty(max(1, L.linear_workspace_bytes(M, wl.n1, wl.n2, desc)), dtype=torch.uint8,
                     device=dev)
    Xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((M,), dtype=torch.float32, device=dev)
    tq_ws = torch.empty(max(1, L.transform_quant_workspace_bytes(M, wl.n1, wl.n2, False)),
                        dtype=torch.uint8, device=dev)
    g_ws = torch.empty(max(1, L.gemm_workspace_bytes(M, desc)), dtype=torch.uint8, device=dev)
    f6 = args.gemm == "f6"
    if f6:
        # offline: the packed weights to the fp6 layout (exact), one per copy
        w6 = [L.pack_weights_f6(desc, Wq, zw) for (_, Wq, _, zw) in packs]
        ws = torch.empty(max(1, L.linear_f6_workspace_bytes(M, wl.n1, wl.n2, desc)),
                         dtype=torch.uint8, device=dev)
        g_ws = torch.empty(max(1, L.gemm_f6_workspace_bytes(M, desc)), dtype=torch.uint8,
                           device=dev)
        torch.cuda.synchronize()

    # single-kernel decode (one launch per layer), on request
    single = False
    sync = dws = None
    if args.path == "single" and M <= 16:
        sync = L.decode_sync_buffer(dev)
        dws = torch.empty(max(1, L.linear_decode_workspace_bytes(M, wl.n1, wl.n2)),
                          dtype=torch.uint8, device=dev)
        _, Wq, sw, zw = packs[0]
        L.linear_decode(X, P1, P2, desc, Wq, sw, zw, sync=sync, steps=steps, per_channel=pc,
                        out=Y, ws=dws)
        torch.cuda.synchronize()
        single = True
    elif args.path == "single":
        raise SystemExit("--path single needs M <= 16")

    def decode_call(i):
        _, Wq, sw, zw = packs[i % copies]
        L.linear_decode(X, P1, P2, desc, Wq, sw, zw, sync=sync, steps=steps, per_channel=pc,
                        out=Y, ws=dws)

    def step(i):
        _, Wq, sw, zw = packs[i % copies]
        if single:
            decode_call(i)
        elif static:
            L.linear_static(X, P1, P2, steps, pc, desc, Wq, sw, zw, out=Y, ws=ws)
        elif f6:
            L.linear_f6(X, P1, P2, desc, w6[i % copies], sw, out=Y, ws=ws)
        else:
            L.linear_bits(X, P1, P2, args.bits, desc, Wq, sw, zw, out=Y, ws=ws)

    def gemm_call(i):
        _, Wq, sw, zw = packs[i % copies]
        if f6:
            L.gemm_f6(Xq, sx, desc, w6[i % copies], sw, out=Y, ws=g_ws)
        else:
            L.gemm(Xq, sx, desc, Wq, sw, zw, out=Y, ws=g_ws)

    def act(i):
        if static:
            L.transform_quant_static(X, P1, P2, steps, pc, out=(Xq, sx), ws=tq_ws)
        else:
            L.transform_quant_bits(X, P1, P2, args.bits, out=(Xq, sx), ws=tq_ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps

    # per-kernel durations: each kernel launched back to back `steps` times
    # between two HIP events on the launch stream (torch's current stream,
    # which the binding uses); the GEMM reads the activations the transform
    # left in Xq / sx and rotates the weight copies like the timed steps
    for i in range(args.warmup):
        act(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        act(i)
    e1.record()
    torch.cuda.synchronize()
    tq_us = e0.elapsed_time(e1) * 1e3 / args.steps
    for i in range(args.warmup):
        gemm_call(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        gemm_call(i)
    e1.record()
    torch.cuda.synchronize()
    gemm_us = e0.elapsed_time(e1) * 1e3 / args.steps

    single_us = None
    if single:
        for i in range(args.warmup):
            decode_call(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            decode_call(i)
        e1.record()
        torch.cuda.synchronize()
        single_us = e0.elapsed_time(e1) * 1e3 / args.steps
        if int(sync[L.DECODE_SYNC_ERROR_WORD].item()) != 0:
            raise SystemExit("the single-kernel decode timed out waiting for its activations")

    dist = event_stats(decode_call if single else gemm_call, max(20, args.steps))

    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12
    tq_bytes = 2 * M * K + M * K // 2 + 4 * M + 4 * (wl.n1 * wl.n1 + wl.n2 * wl.n2)
    tq_flops = 2.0 * M * K * (wl.n1 + wl.n2)
    transform = {"us": round(tq_us, 2), "bytes": tq_bytes, "flops": tq_flops,
                 "achieved_GBps": round(tq_bytes / (tq_us * 1e-6) / 1e9, 1),
                 "achieved_GFLOPps": round(tq_flops / (tq_us * 1e-6) / 1e9, 1),
                 "t_at_hbm_us": round(tq_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                 "t_at_fp32_vector_us": round(tq_flops / 157.3e12 * 1e6, 2)}
    if single:
        # the one kernel of the layer: weights, scales, activations in and out
        gb = layer_bytes(wl, M)
        achieved = gb / (single_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        roof["kernel"] = f"k_linear_dec<n1 {wl.n1}, 8 waves, depth 12>"
        roof["kernel_us"] = round(single_us, 2)
        roof["traffic"] = traffic_from_profiles("linear_dec", wl.name, "linear_decode.hip")
    elif decode:
        gb = gemm_bytes(wl, M)
        achieved = gb / (gemm_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
        roof["kernel"] = L.gemm_kernel_name(M, desc)
        roof["kernel_us"] = round(gemm_us, 2)
        roof["traffic"] = traffic_from_profiles("gemm", wl.name)
    elif f6:
        # the w4a4_gemm_f6 call: activations to the fp6 layout, then the product
        achieved = ops / (gemm_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP6_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_FP6_TOPS, 4)}
        roof["kernel"] = "w4a4_gemm_f6 = k_f6_convert + " + L.gemm_f6_kernel_name(M, desc)
        roof["kernel_us"] = round(gemm_us, 2)
        roof["traffic"] = traffic_from_profiles("gemm_f6", wl.name, "gemm_f6.hip")
    else:
        achieved = ops / (gemm_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4)}
        roof["kernel"] = L.gemm_kernel_name(M, desc)
        roof["kernel_us"] = round(gemm_us, 2)
        roof["traffic"] = traffic_from_profiles("gemm", wl.name)
    roof["timing"] = ("mean over HIP events around back-to-back launches on the launch stream; "
                      "per_launch_us from events around each launch")
    roof["per_launch_us"] = dist

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp6 E2M3 MFMA on the exact int4 codes (v/2), fp32 acc, fp32 transform" if f6
                  else "int8 MFMA/int32 acc (int4 codes), fp32 transform"),
        "data": "synthetic (seeded; LLaMA-shaped, outlier channels and pivot token)",
        "config": {"workload": wl.description, "name": wl.name, "M": M, "K": K, "N": N,
                   "n1": wl.n1, "n2": wl.n2, "group_size": wl.group_size,
                   "asymmetric_weights": wl.asymmetric, "weight_copies_rotated": copies,
                   "act_quant": args.act_quant, "bits": args.bits, "gemm": args.gemm},
        "us_per_layer": round(t_step * 1e6, 2),
        "path": ("single-kernel decode (w4a4_linear_decode)" if single else
                 "transform + fp6 conversion + product (w4a4_linear_f6)" if f6 else
                 "two launches (w4a4_linear)"),
        "transform_quant_us": round(tq_us, 2),
        "transform_quant": transform,
        "gemm_us": round(gemm_us, 2),
        "single_kernel_us": None if single_us is None else round(single_us, 2),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds, args.act_quant, args.bits)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# decode attention over the INT4 KV cache
# ---------------------------------------------------------------------------
ATTN_BYTES_PER_TOKEN_HEAD = 64 + 64 + 4 + 4      # key and value codes, two fp32 scales


def attn_bytes(wl, lengths):
    """Algorithmic bytes of one w4a4_attn_decode call: the cached codes and
    scales of every context token and KV head, the fp16 queries and outputs,
    and the fp32 query factor."""
    tok = int(np.sum(lengths))
    return (tok * wl.heads_kv * ATTN_BYTES_PER_TOKEN_HEAD + 2 * 2 * wl.batch * wl.heads_q * 128
            + 4 * 128 * 128)


def attn_cpu_baseline(wl, st, budget_s):
    """The oracle's decode attention on whole sequences until `budget_s`,
    projected to the layer by context tokens."""
    import math
    from oracle import kv_oracle as KV
    from workloads import kv as WKV
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    sm = 1.0 / math.sqrt(128)
    done_tok, t_used, seqs = 0, 0.0, 0
    for b in range(wl.batch):
        L = int(st["lengths"][b])
        k, v = WKV.make_history(wl, b, L, st["outliers"])
        oc = KV.KvCache(1, wl.heads_kv, wl.max_seq, 128)
        KV.kv_append(oc, k, v, [0], [0], [0, L], st["P_h"], st["P_v"])   # untimed
        t0 = time.perf_counter()
        KV.attention_decode(st["q"][b:b + 1], oc, np.array([L]), st["P_h"], sm)
        t_used += time.perf_counter() - t0
        done_tok += L
        seqs += 1
        if t_used >= budget_s:
            break
    total_tok = int(np.sum(st["lengths"]))
    t_layer = t_used / done_tok * total_tok
    ops = 4.0 * total_tok * wl.heads_q * 128
    return {"value": ops / t_layer / 1e12, "unit": "TOPS", "cores": int(threads),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"decode attention of {seqs} of the {wl.batch} sequences ({done_tok} context "
                      f"tokens, caches built untimed), {t_used:.1f} s, projected to all "
                      f"{total_tok} tokens",
            "us_per_layer": t_layer * 1e6}


def attn_main(args):
    import math
    import torch
    import w4a4_post_quantized_amd as L
    from workloads import kv as WKV

    wl = WKV.get_kv(args.workload)
    st = WKV.make_kv_static(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, S = wl.batch, wl.heads_q, wl.heads_kv, wl.max_seq
    lengths = st["lengths"]                      # contexts including the step's new token
    cache = L.KvCache(B, Hkv, S, dev)
    P_h = torch.from_numpy(st["P_h"]).to(dev)
    P_v = torch.from_numpy(st["P_v"]).to(dev)
    # the cached history (positions 0 .. L-2), drawn on the GPU with the
    # workload's distribution: N(0,1), keys with x8 outlier channels per head
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed)
    hist = (lengths - 1).astype(np.int64)
    T = int(hist.sum())
    kscale = torch.ones((Hkv, 128), device=dev)
    for h in range(Hkv):
        kscale[h, torch.from_numpy(st["outliers"][h]).to(dev)] = wl.outlier_scale
    k = (torch.randn((T, Hkv, 128), generator=g, device=dev) * kscale).half()
    v = torch.randn((T, Hkv, 128), generator=g, device=dev).half()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(hist)]).astype(np.int32)).to(dev)
    seqs = torch.arange(B, dtype=torch.int32, device=dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=dev)
    L.kv_append(k, v, seqs, zeros, cu, P_h, P_v, cache)
    torch.cuda.synchronize()
    del k, v

    # prefill append rate: one 2048-token segment of one sequence
    kp = torch.randn((2048, Hkv, 128), generator=g, device=dev).half()
    vp = torch.randn((2048, Hkv, 128), generator=g, device=dev).half()
    cup = torch.tensor([0, 2048], dtype=torch.int32, device=dev)
    one = torch.tensor([B - 1], dtype=torch.int32, device=dev)
    zero1 = torch.zeros(1, dtype=torch.int32, device=dev)
    pre_cache = L.KvCache(1, Hkv, 2048, dev)
    for _ in range(3):
        L.kv_append(kp, vp, zero1, zero1, cup, P_h, P_v, pre_cache)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        L.kv_append(kp, vp, zero1, zero1, cup, P_h, P_v, pre_cache)
    e1.record()
    torch.cuda.synchronize()
    prefill_us = e0.elapsed_time(e1) * 1e3 / 20
    prefill_bytes = 2 * 2048 * Hkv * 128 * 2 + 2048 * Hkv * ATTN_BYTES_PER_TOKEN_HEAD
    del kp, vp, pre_cache, one

    # the decode step: append the new token at position L-1, attend over L
    kn, vn = WKV.make_new_tokens(wl, st["outliers"])
    kn = torch.from_numpy(kn).to(dev)
    vn = torch.from_numpy(vn).to(dev)
    pos = torch.from_numpy(hist.astype(np.int32)).to(dev)
    cun = torch.arange(B + 1, dtype=torch.int32, device=dev)
    q = torch.from_numpy(st["q"]).to(dev)
    lens = torch.from_numpy(lengths.astype(np.int32)).to(dev)
    Pinv = L.kv_query_factor(P_h)
    sm = 1.0 / math.sqrt(128)
    out = torch.empty((B, Hq, 128), dtype=torch.float16, device=dev)
    ws = torch.empty(max(1, L.attn_decode_workspace_bytes(B, Hq, Hkv, S)), dtype=torch.uint8,
                     device=dev)

    def attend(i):
        L.attn_decode(q, Pinv, cache, lens, sm, out=out, ws=ws)

    def step(i):
        L.kv_append(kn, vn, seqs, pos, cun, P_h, P_v, cache)
        attend(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps

    for i in range(args.warmup):
        attend(i)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        attend(i)
    e1.record()
    torch.cuda.synchronize()
    attn_us = e0.elapsed_time(e1) * 1e3 / args.steps
    e0.record()
    for i in range(args.steps):
        L.kv_append(kn, vn, seqs, pos, cun, P_h, P_v, cache)
    e1.record()
    torch.cuda.synchronize()
    append_us = e0.elapsed_time(e1) * 1e3 / args.steps
    dist = event_stats(attend, max(20, args.steps))

    gb = attn_bytes(wl, lengths)
    achieved = gb / (attn_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "kernel": "w4a4_attn_decode (k_rows_xform + k_attn_partial + k_attn_combine)",
            "kernel_us": round(attn_us, 2), "bytes": gb,
            "bytes_per_unit": f"{ATTN_BYTES_PER_TOKEN_HEAD} B per cached (token, KV head)",
            "traffic": traffic_from_profiles("attn", wl.name, "attention.hip"),
            "timing": "mean over HIP events around back-to-back calls on the launch stream; "
                      "per_launch_us from events around each call",
            "per_launch_us": dist}
    ops = 4.0 * float(np.sum(lengths)) * Hq * 128
    res = {
        "metric": METRIC, "value": round(ops / t_step / 1e12, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int4 KV codes, fp16 MFMA with exact hi/lo operands, fp32 accumulation",
        "data": "synthetic (seeded; N(0,1) queries, keys with x8 outlier channels, values; "
                "ragged contexts)",
        "config": {"workload": wl.description, "name": wl.name, "batch": B, "heads_q": Hq,
                   "heads_kv": Hkv, "head_dim": 128, "max_seq": S,
                   "context_tokens": int(np.sum(lengths))},
        "us_per_layer": round(t_step * 1e6, 2),
        "path": "w4a4_kv_append (decode tokens) + w4a4_attn_decode",
        "attn_us": round(attn_us, 2), "append_decode_us": round(append_us, 2),
        "append_prefill_2048": {"us": round(prefill_us, 2), "bytes": prefill_bytes,
                                "achieved_GBps": round(prefill_bytes / (prefill_us * 1e-6) / 1e9, 1)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = attn_cpu_baseline(wl, st, args.cpu_seconds)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
# ternary-weight decode product
# ---------------------------------------------------------------------------
TERN_BYTES_PER_WEIGHT = 0.25 + 4.0 / 128       # 2-bit code + one 32-bit word per 128


def tern_bytes(wl):
    """Algorithmic bytes of one w4a4_ternary_gemm call: the packed codes and
    block parameters, the fp16 activations and the fp16 outputs."""
    G = wl.K // 128
    return wl.N * wl.K // 4 + 4 * wl.N * G + 2 * wl.M * wl.K + 2 * wl.M * wl.N


def tern_cpu_baseline(wl, X, budget_s):
    """The oracle's ternary layer on chunks of output columns until `budget_s`
    of layer time (each chunk ternarized by the oracle first, untimed; the
    ternarization is offline work), projected to all N columns."""
    from oracle import ternary_oracle as TO
    from workloads import ternary as WT
    threads = os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())
    chunk = 256
    done, t_used, wall0 = 0, 0.0, time.perf_counter()
    for r0 in range(0, wl.N, chunk):
        rows = np.arange(r0, min(wl.N, r0 + chunk))
        r = TO.itf_ternarize(WT.make_tern_weights(wl, rows=rows))        # untimed
        t0 = time.perf_counter()
        TO.ternary_linear(X, r)
        t_used += time.perf_counter() - t0
        done += rows.size
        if t_used >= budget_s or time.perf_counter() - wall0 >= 3 * budget_s:
            break
    t_layer = t_used / done * wl.N
    ops = 2.0 * wl.M * wl.N * wl.K
    return {"value": ops / t_layer / 1e12, "unit": "TOPS", "cores": int(threads),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"the float64 layer on {done} of the {wl.N} output columns (weights "
                      f"ternarized by the oracle untimed), {t_used:.2f} s, projected to all "
                      f"columns",
            "us_per_layer": t_layer * 1e6}


def tern_main(args):
    import torch
    import w4a4_post_quantized_amd as L
    from workloads import ternary as WT

    wl = WT.get_tern(args.workload)
    inp = WT.make_tern_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    X = torch.from_numpy(inp["X"]).to(dev)
    Wt = torch.from_numpy(inp["Wt"]).to(dev)
    del inp["Wt"]
    Tq, am = L.pack_ternary(Wt)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    del Wt
    wbytes = Tq.numel() + 4 * am.numel()
    copies = max(3, -(-MALL_BYTES // wbytes) + 1)
    packs = [(Tq, am)] + [(Tq.clone(), am.clone()) for _ in range(copies - 1)]
    Y = torch.empty((wl.M, wl.N), dtype=torch.float16, device=dev)
    ws = torch.empty(max(1, L.ternary_gemm_workspace_bytes(wl.M, wl.N, wl.K)), dtype=torch.uint8,
                     device=dev)

    def step(i):
        t, a = packs[i % copies]
        L.ternary_gemm(X, t, a, wl.N, out=Y, ws=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / args.steps
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    call_us = e0.elapsed_time(e1) * 1e3 / args.steps
    dist = event_stats(step, max(20, args.steps))

    gb = tern_bytes(wl)
    achieved = gb / (call_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "kernel": "w4a4_ternary_gemm (k_tern_rowsum + k_tern_gemm + k_tern_reduce)",
            "kernel_us": round(call_us, 2), "bytes": gb,
            "bytes_per_unit": f"{TERN_BYTES_PER_WEIGHT} B per weight (2-bit code, 32-bit "
                              "(alpha, mu) word per 128) plus fp16 X and Y",
            "traffic": traffic_from_profiles("tern", wl.name, "ternary.hip"),
            "timing": "mean over HIP events around back-to-back calls on the launch stream, "
                      f"{copies} weight copies rotated past the 256 MiB Infinity Cache; "
                      "per_launch_us from events around each call",
            "per_launch_us": dist}
    ops = 2.0 * wl.M * wl.N * wl.K
    res = {
        "metric": METRIC, "value": round(ops / t_step / 1e12, 3), "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "ternary weights (2-bit codes), fp16 activations, fp16 MFMA, fp32 accumulation",
        "data": "synthetic (seeded; weights with per-row scales, per-block offsets and x8 "
                "outliers; decode activations)",
        "config": {"workload": wl.description, "name": wl.name, "M": wl.M, "K": wl.K,
                   "N": wl.N, "block": 128, "weight_copies_rotated": copies},
        "us_per_layer": round(t_step * 1e6, 2),
        "path": "w4a4_ternary_gemm",
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = tern_cpu_baseline(wl, inp["X"], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
