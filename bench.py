"""Benchmark of the int4 routed-expert MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L] [--no-graph]
                    [--no-prefill] [--no-quantizer] [--no-cache] [--cache-slots S]
                    [--no-cpu-baseline]

A step is one pass of the whole layer -- route, batch-union, expert FFN,
combine -- over one batch of synthetic tokens, with every input already
resident in HBM.  The headline is the 1-token decode step of the layer shaped
like the pages' GLM-5.2 layer (d=6144, f=2048, 256 routed experts top-8 plus
one shared expert, int4 gs64 with fp16 scales; every expert a 20,054,016-byte
block): effective expert-weight GB/s = (active experts + shared) * block bytes
per step / step time.  Consecutive steps run on different copies of the layer
(``--layers``, default 8, ~41 GB of HBM) and different token batches, the way
consecutive layers of a model follow each other, so no step finds the
previous step's experts in the 256 MB Infinity Cache.  Batches of at most 8
tokens run the layer as the one call moe_layer_decode (four launches); the
same step through the separate calls (moe_route_union, moe_expert_ffn,
moe_combine: five launches) is timed too and reported beside it.

The same run also reports the 2048-token prefill step of that layer (Zipf
router bias, bf16 MFMA path) as tokens/s, the roofline of the dominant
kernel (the expert FFN: HBM bytes for decode), timed with HIP events on the
launch stream, the int4 quantiser, 1-token decode through a per-layer HBM
expert cache whose misses stream from pinned host memory, and the CPU oracle
timed on a bounded sample on the host cores.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
METRIC = "decode int4 expert GB/s (% HBM peak); prefill tokens/s per MoE layer"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=8, help="layer copies rotated in HBM")
    ap.add_argument("--tokens", type=int, default=1, help="decode batch (1 or 8)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graphs")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-cache", action="store_true", help="skip the expert-cache leg")
    ap.add_argument("--cache-slots", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--no-batch8", action="store_true",
                    help="skip the 8-token decode leg (run with the 1-token headline)")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the MXFP4 legs (decode FFN, and the prefill step unless --no-prefill)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured HBM copy/read and bf16 GEMM rates")
    ap.add_argument("--counters", action="store_true",
                    help="only run what the HBM-traffic counter passes measure: a 1 GiB device "
                         "copy (calibration) and 20 decode expert-FFN launches")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(one MI355X per process, no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import synth
    import int4_routed_expert_logits_amd as moe
    from int4_routed_expert_logits_amd.layer import LayerBuffers, run_layer, run_layer_decode

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    moe.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.counters:
        return counter_workload(args, torch, moe, synth, LayerBuffers, run_layer, dev)

    # ------------------------------------------------------------------ data
    t0 = time.time()
    L = synth.make_layer(4)
    sh = moe.shape_of(L.shape)
    bb = L.expert_bytes
    # canonical blocks -> packed blocks (the one-time conversion), on the GPU
    src = torch.from_numpy(L.experts).to(dev)
    experts = [torch.empty_like(src)]
    moe.moe_pack_experts(sh, L.shape.n_experts, src, experts[0])
    del src
    src = torch.from_numpy(L.shared[None]).to(dev)
    shared = [torch.empty_like(src)[0]]
    moe.moe_pack_experts(sh, 1, src, shared[0])
    del src
    for _ in range(1, args.layers):
        experts.append(experts[0].clone())
        shared.append(shared[0].clone())
    w_router = torch.from_numpy(L.w_router).to(dev)
    T = args.tokens
    nb = args.layers
    xs = []
    for b in range(nb):
        bits, _ = synth.make_tokens(4, T, batch=b)
        xs.append(torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16))
    torch.cuda.synchronize()
    log(f"decode data ready in {time.time() - t0:.1f}s: {args.layers} layer copies x "
        f"{experts[0].numel() / 1e9:.2f} GB, {nb} token batches of {T}")

    DEC = moe.MOE_PATH_DECODE_F32
    bufs = [LayerBuffers.allocate(sh, T, DEC) for _ in range(nb)]

    def step_calls(i):  # moe_route_union, moe_expert_ffn, moe_combine
        j = i % nb
        run_layer(xs[j], w_router, None, experts[j % args.layers], shared[j % args.layers], bufs[j])

    def step_one_call(i):  # moe_layer_decode
        j = i % nb
        run_layer_decode(xs[j], w_router, None, experts[j % args.layers], shared[j % args.layers],
                         bufs[j])

    one_call = T <= 8
    step = step_one_call if one_call else step_calls

    # --------------------------------------------------- per-kernel timing (events)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n_kt = max(args.steps, 2 * nb)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_kt)]
    for i in range(n_kt):
        j = i % nb
        b = bufs[j]
        moe.moe_route(sh, xs[j], w_router, None, b.topk_idx, b.topk_w, b.workspace)
        moe.moe_union(sh, T, b.topk_idx, b.counts, b.offsets, b.perm, b.inv_perm, b.active, b.n_active)
        ev[i][0].record(stream)
        moe.moe_expert_ffn(sh, xs[j], experts[j % args.layers], shared[j % args.layers], b.offsets,
                           b.perm, b.active, b.n_active, DEC, b.y, b.y_shared, b.ffn_workspace)
        ev[i][1].record(stream)
        moe.moe_combine(sh, b.y, b.y_shared, b.inv_perm, b.topk_w, b.out)
    torch.cuda.synchronize()
    ffn_ms = np.array([s.elapsed_time(e) for s, e in ev])
    active_per_batch = [int(b.n_active.item()) for b in bufs]
    bytes_per_batch = [(a + 1) * bb for a in active_per_batch]
    ffn_bytes = np.array([bytes_per_batch[i % nb] for i in range(n_kt)], dtype=np.float64)
    kern_gbps = float(np.sum(ffn_bytes) / (np.sum(ffn_ms) * 1e-3) / 1e9)
    log(f"expert FFN kernel: mean {ffn_ms.mean() * 1e3:.1f} us, median {np.median(ffn_ms) * 1e3:.1f} us, "
        f"{kern_gbps:.0f} GB/s over {n_kt} launches")

    # --------------------------------------------------------- timed region
    def timed(step):
        """Exactly args.steps steps, timed with HIP events on the launch
        stream (synchronised on both sides); returns (ms per step, steps,
        per-step us percentiles over >= 64 separately timed graph replays)."""
        steps = args.steps
        dist = None
        if not args.no_graph:
            s = torch.cuda.Stream()
            s.wait_stream(stream)
            with torch.cuda.stream(s):
                for i in range(nb):       # warm the capture stream
                    step(i)
            stream.wait_stream(s)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(nb):
                    step(i)
            rest = None
            if steps % nb:
                rest = torch.cuda.CUDAGraph()
                with torch.cuda.graph(rest):
                    for i in range(steps % nb):
                        step(i)
            for _ in range(max(1, args.warmup // nb)):
                graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps // nb):
                graph.replay()
            if rest is not None:
                rest.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            elapsed_ms = e0.elapsed_time(e1)
            # the distribution: graph replays of nb steps, each event-timed
            reps = 64
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(reps)]
            for a_, b_ in evs:
                a_.record(stream)
                graph.replay()
                b_.record(stream)
            torch.cuda.synchronize()
            per = np.array([a_.elapsed_time(b_) for a_, b_ in evs]) * 1e3 / nb
            dist = {"us_p10": round(float(np.percentile(per, 10)), 2),
                    "us_p50": round(float(np.percentile(per, 50)), 2),
                    "us_p90": round(float(np.percentile(per, 90)), 2),
                    "replays": reps, "steps_per_replay": nb}
            del graph, rest
        else:
            for i in range(args.warmup):
                step(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                step(i)
            e1.record(stream)
            torch.cuda.synchronize()
            elapsed_ms = e0.elapsed_time(e1)
        return elapsed_ms / steps, steps, dist

    step_bytes = float(np.mean(bytes_per_batch))
    graph = not args.no_graph
    ms_calls, steps, dist_calls = timed(step_calls)
    log(f"decode step, separate calls: {ms_calls * 1e3:.1f} us, "
        f"{step_bytes / (ms_calls * 1e-3) / 1e9:.0f} GB/s ({'graph' if graph else 'eager'}) {dist_calls}")
    ms_per_step, dist = ms_calls, dist_calls
    if one_call:
        ms_per_step, steps, dist = timed(step_one_call)
        log(f"decode step, moe_layer_decode: {ms_per_step * 1e3:.1f} us, "
            f"{step_bytes / (ms_per_step * 1e-3) / 1e9:.0f} GB/s {dist}")
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"decode, {T} token(s) per step, layer d=6144 f=2048, 256 routed experts "
                        f"top-8 + 1 shared, int4 gs64 fp16 scales (20,054,016 B per expert)",
            "tokens_per_step": T,
            "layer_copies_rotated": args.layers,
            "launch": ("hip graph" if graph else "eager") +
                      (", moe_layer_decode (4 launches)" if one_call
                       else ", moe_route_union + moe_expert_ffn + moe_combine (5 launches)"),
            "separate_calls_us_per_step": round(ms_calls * 1e3, 2),
            "step_us_distribution": dist,
            "timing": "HIP events on the launch stream around exactly `steps` steps "
                      "(graph replays of 8 steps plus one of the remainder)",
            "expert_blocks_per_step": round(step_bytes / bb, 3),
            "hbm_pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "moe_expert_ffn (decode)",
            "achieved": round(kern_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic(),
            "algorithmic_bytes_per_launch": step_bytes,
            "avg_launch_us": round(float(ffn_ms.mean()) * 1e3, 2),
        },
    }

    # ------------------------------------------ decode batch of 8 tokens (one call)
    if T == 1 and not args.no_batch8:
        result["decode_8_tokens"] = bench_decode_batch(args, torch, moe, synth, LayerBuffers,
                                                       run_layer_decode, run_layer, sh, experts,
                                                       shared, w_router, bb, 8)
        # a multi-token-prediction verify batch (the pages: 2.2-2.8 tokens per forward)
        result["decode_3_tokens_mtp_verify"] = bench_decode_batch(
            args, torch, moe, synth, LayerBuffers, run_layer_decode, run_layer, sh, experts,
            shared, w_router, bb, 3)

    # ----------------------------------------------------- MXFP4 decode FFN
    if T == 1 and not args.no_mxfp4:
        result["mxfp4_decode"], mx_pre = bench_mxfp4(args, torch, moe, synth, LayerBuffers,
                                                     run_layer, w_router, xs, dev)
        if mx_pre is not None:
            result["mxfp4_prefill"] = mx_pre

    # ------------------------------------------------------- measured peaks
    if not args.no_peaks:
        peaks = measured_peaks(torch, dev)
        peaks.update(stream_read_peak(torch, moe, experts, shared, bufs, bb, dev))
        result["measured_peaks"] = peaks
        result["roofline"]["frac_of_measured_copy"] = round(kern_gbps / peaks["torch_copy_gbps"], 4)
        result["roofline"]["attainable_read_gbps"] = peaks["stream_read_gbps"]
        result["roofline"]["frac_of_attainable"] = round(kern_gbps / peaks["stream_read_gbps"], 4)

    # --------------------------------------------------------------- prefill
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args, torch, moe, synth, LayerBuffers, run_layer, sh, experts[0], shared[0], w_router, dev)
    if "measured_peaks" in result:
        for leg in ("prefill", "mxfp4_prefill"):
            if "roofline" in result.get(leg, {}):
                pr = result[leg]["roofline"]
                pr["frac_of_measured_gemm"] = round(
                    pr["achieved"] / result["measured_peaks"]["torch_matmul_bf16_tflops"], 4)

    # ------------------------------------------------------------ quantiser
    if not args.no_quantizer:
        result["quantizer"] = bench_quantizer(torch, moe, dev)

    # --------------------------------------------------------- expert cache
    if not args.no_cache:
        result["expert_cache"] = bench_cache(args, torch, moe, synth, sh, experts[0], shared[0],
                                             w_router, dev)

    # ----------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(L, bb)

    print(json.dumps(result), flush=True)
    return 0


def bench_decode_batch(args, torch, moe, synth, LayerBuffers, run_layer_decode, run_layer, sh,
                       experts, shared, w_router, bb, T):
    """Decode steps of T tokens (8: the 19 MB-expert layer's second decode
    batch size; 3: a multi-token-prediction verify batch), each form of the
    step -- the one call moe_layer_decode and the separate calls
    moe_route_union + moe_expert_ffn + moe_combine -- captured in a HIP graph
    over the rotating layer copies and timed with HIP events; expert bytes =
    (distinct routed experts + shared) x block."""
    dev = w_router.device
    stream = torch.cuda.current_stream()
    nb = len(experts)
    xs, bufs = [], []
    for b in range(nb):
        bits, _ = synth.make_tokens(4, T, batch=100 + b)
        xs.append(torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16))
        bufs.append(LayerBuffers.allocate(sh, T, moe.MOE_PATH_DECODE_F32))

    def time_form(run):
        def step(i):
            j = i % nb
            run(xs[j], w_router, None, experts[j], shared[j], bufs[j])

        for i in range(nb):
            step(i)
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for i in range(nb):
                step(i)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(nb):
                step(i)
        reps = max(8, args.steps // nb)
        for _ in range(max(1, args.warmup // nb)):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        del graph
        return e0.elapsed_time(e1) / (reps * nb)

    ms = time_form(run_layer_decode)
    ms_sep = time_form(run_layer)
    blocks = [int(b.n_active.item()) + 1 for b in bufs]
    step_bytes = float(np.mean(blocks)) * bb
    gbps = step_bytes / (ms * 1e-3) / 1e9
    log(f"decode step, {T} tokens: moe_layer_decode {ms * 1e3:.1f} us, separate calls "
        f"{ms_sep * 1e3:.1f} us; {gbps:.0f} GB/s ({np.mean(blocks):.1f} expert blocks per step), "
        f"{T / (ms * 1e-3):.0f} tokens/s")
    return {
        "value": round(gbps, 2),
        "unit": "GB/s",
        "us_per_step": round(ms * 1e3, 2),
        "separate_calls_us_per_step": round(ms_sep * 1e3, 2),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "expert_blocks_per_step": round(float(np.mean(blocks)), 2),
        "hbm_pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "workload": f"decode, {T} tokens per step, same layer, no router bias, hip graph over "
                    f"{nb} layer copies; value from moe_layer_decode",
    }


def bench_mxfp4(args, torch, moe, synth, LayerBuffers, run_layer, w_router, xs, dev, copies=4):
    """The expert FFN (moe_expert_ffn) on MXFP4 experts of the same geometry
    (shape group 32: E2M1 codes, one E8M0 byte per 32; the same 20,054,016
    bytes per expert): the decode path in 1-token steps rotating over
    `copies` layer copies, each launch event-timed like the int4 FFN, then
    (unless --no-prefill) the 2048-token prefill step as for int4 experts.
    Returns (decode result, prefill result or None)."""
    L = synth.make_layer(4, fmt="mxfp4")
    s = L.shape
    sh = moe.Shape(s.d, s.f, s.n_experts, s.top_k, 32, s.f_shared)
    bb = L.expert_bytes
    src = torch.from_numpy(L.experts).to(dev)
    experts = [torch.empty_like(src)]
    moe.moe_pack_experts(sh, s.n_experts, src, experts[0])
    del src
    src = torch.from_numpy(L.shared[None]).to(dev)
    shared = [torch.empty_like(src)[0]]
    moe.moe_pack_experts(sh, 1, src, shared[0])
    del src, L
    for _ in range(1, copies):
        experts.append(experts[0].clone())
        shared.append(shared[0].clone())
    DEC = moe.MOE_PATH_DECODE_F32
    nb = len(xs)
    bufs = [LayerBuffers.allocate(sh, 1, DEC) for _ in range(nb)]
    for j in range(nb):
        run_layer(xs[j], w_router, None, experts[j % copies], shared[j % copies], bufs[j])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    n = max(args.steps, 2 * nb)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(args.warmup + n):
        j = i % nb
        b = bufs[j]
        if i >= args.warmup:
            ev[i - args.warmup][0].record(stream)
        moe.moe_expert_ffn(sh, xs[j], experts[i % copies], shared[i % copies], b.offsets, b.perm,
                           b.active, b.n_active, DEC, b.y, b.y_shared, b.ffn_workspace)
        if i >= args.warmup:
            ev[i - args.warmup][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(e) for a, e in ev])
    blocks = [int(b.n_active.item()) + 1 for b in bufs]
    step_bytes = float(np.mean(blocks)) * bb
    gbps = step_bytes / (ms.mean() * 1e-3) / 1e9
    log(f"MXFP4 expert FFN kernel: mean {ms.mean() * 1e3:.1f} us, {gbps:.0f} GB/s "
        f"({np.mean(blocks):.1f} blocks of {bb} B)")
    del bufs
    pre = None
    if not args.no_prefill:
        pre = bench_prefill(args, torch, moe, synth, LayerBuffers, run_layer, sh, experts[0],
                            shared[0], w_router, dev, fmt="mxfp4")
    del experts, shared
    torch.cuda.empty_cache()
    return {
        "value": round(gbps, 1),
        "unit": "GB/s",
        "avg_launch_us": round(float(ms.mean()) * 1e3, 2),
        "hbm_pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {"bound": "hbm", "kernel": "moe_expert_ffn (decode, MXFP4)",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode", "mxfp4"),
                     "algorithmic_bytes_per_launch": step_bytes},
        "workload": "moe_expert_ffn decode path, 1 token, MXFP4 experts of the d=6144 f=2048 "
                    f"layer (E2M1 + E8M0 per 32, {bb} B per expert), {copies} layer copies rotated",
    }, pre


def measured_peaks(torch, dev, reps=10):
    """What plain library work reaches on this GPU, beside the published
    peaks: a 1 GiB device copy (read + write bytes counted), a float32 sum
    over 1 GiB (read only), and an 8192^3 bf16 matrix product through
    torch.matmul (the vendor BLAS)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    af = a.view(torch.float32)

    def rate(fn, work):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return work / (e0.elapsed_time(e1) * 1e-3 / reps)

    copy = rate(lambda: b.copy_(a), 2.0 * n) / 1e9
    read = rate(lambda: af.sum(), float(n)) / 1e9
    del a, b, af
    m = 8192
    x = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    w = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    gemm = rate(lambda: torch.matmul(x, w), 2.0 * m * m * m) / 1e12
    del x, w
    log(f"measured: device copy {copy:.0f} GB/s, 1 GiB read {read:.0f} GB/s, "
        f"bf16 GEMM {gemm:.0f} TFLOP/s")
    return {
        "torch_copy_gbps": round(copy, 1),
        "torch_sum_read_gbps": round(read, 1),
        "torch_matmul_bf16_tflops": round(gemm, 1),
        "how": "torch copy_ of 1 GiB (read + write bytes counted), torch sum over 1 GiB of "
               "float32 (a library reduction, below what a plain streaming read reaches), "
               "torch.matmul 8192x8192x8192 bf16 (vendor BLAS); 10 timed repetitions each",
    }


def stream_read_peak(torch, moe, experts, shared, bufs, bb, dev, rounds=8):
    """What a plain read-only kernel attains on the decode step's own bytes:
    moe_measure_stream_read over the shared block and the routed blocks of
    each token batch (the 180.5 MB the decode FFN streams), rotating over the
    layer copies as the timed steps do, for a few grid sizes; the best
    (event-timed, mean over the rounds) is the attainable rate."""
    nb = len(bufs)
    sets = []
    for j in range(nb):
        act = bufs[j].active.cpu().numpy()
        ids = [int(e) for e in act if e >= 0]
        sets.append([shared[j % len(shared)].data_ptr()] +
                    [experts[j % len(experts)].data_ptr() + e * bb for e in ids])
    sink = torch.empty((1 << 16,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    best, table = 0.0, {}
    for wg in (2304, 4608, 9216, 18432, 36864):
        def run(j):
            moe.moe_measure_stream_read(sets[j], bb, wg, sink)
        for j in range(nb):
            run(j)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(rounds * nb)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            run(i % nb)
            b.record(stream)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        nbytes = np.array([len(sets[i % nb]) * bb for i in range(len(evs))], dtype=np.float64)
        gbps = float(nbytes.sum() / (us.sum() * 1e-6) / 1e9)
        table[wg] = round(gbps, 1)
        best = max(best, gbps)
    log(f"measured: plain read of the decode step's expert blocks {best:.0f} GB/s "
        f"(by workgroups: {table})")
    return {"stream_read_gbps": round(best, 1), "stream_read_by_workgroups": table,
            "stream_read_how": "moe_measure_stream_read over the shared + routed expert blocks "
                               "of each 1-token step (9 x 20,054,016 B), layer copies rotated, "
                               "event-timed; best grid of 2304..36864 workgroups"}


def bench_quantizer(torch, moe, dev, reps=20):
    """The one-time conversion: the three bf16 matrices of one ~19 MB expert
    (W_gate, W_up [2048, 6144], W_down [6144, 2048]) quantised to int4 gs64,
    timed with HIP events on the current stream.  Algorithmic bytes: 2 per
    weight read, 0.5 + 2/64 per weight written."""
    d, f = 6144, 2048
    g = torch.Generator(device=dev).manual_seed(20261205)
    mats = [torch.randn((f, d), generator=g, device=dev).to(torch.bfloat16),
            torch.randn((f, d), generator=g, device=dev).to(torch.bfloat16),
            torch.randn((d, f), generator=g, device=dev).to(torch.bfloat16)]
    outs = [(torch.empty((m.shape[0], m.shape[1] // 2), dtype=torch.uint8, device=dev),
             torch.empty((m.shape[0], m.shape[1] // 64), dtype=torch.float16, device=dev)) for m in mats]

    def run():
        for m, (c, sc) in zip(mats, outs):
            moe.moe_quantize(m, moe.MOE_QUANT_GS64, c, sc)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        run()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    n_w = 3 * d * f
    alg = n_w * 2 + n_w // 2 + n_w // 64 * 2
    gbps = alg / (float(np.median(us)) * 1e-6) / 1e9
    log(f"quantiser: one expert (3 x {f}x{d} bf16) in {np.median(us):.1f} us = {gbps:.0f} GB/s")
    return {
        "value": round(gbps, 1),
        "unit": "GB/s",
        "workload": "int4 gs64 quantisation of one expert's three bf16 matrices (d=6144, f=2048)",
        "us_per_expert": round(float(np.median(us)), 2),
        "roofline": {"bound": "hbm", "kernel": "moe_quantize (gs64)", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": alg},
    }


PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction


def bench_cache(args, torch, moe, synth, sh, experts, shared, w_router, dev, warm=32, steps=64):
    """1-token decode steps through a per-layer cache of --cache-slots
    experts in HBM, the layer's 256 blocks in pinned host memory, Zipf(1.1)
    router bias: tokens/s of the layer, hit rate, and the host -> HBM rate
    of the misses against a plain pinned copy and the PCIe peak."""
    from int4_routed_expert_logits_amd.layer import LayerBuffers
    slots = args.cache_slots
    bb = moe.moe_expert_bytes(sh.d, sh.f, 64)
    host = torch.empty((experts.numel(),), dtype=torch.uint8, pin_memory=True)
    host.copy_(experts.view(-1))
    torch.cuda.synchronize()
    # a plain pinned host -> HBM copy of 1 GiB: the practical link rate
    blk = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    blk.copy_(host[: 1 << 30], non_blocking=True)
    a.record()
    for _ in range(3):
        blk.copy_(host[: 1 << 30], non_blocking=True)
    b.record()
    torch.cuda.synchronize()
    h2d = 3 * (1 << 30) / (a.elapsed_time(b) * 1e-3) / 1e9
    del blk
    dev_slots = torch.empty((slots * bb,), dtype=torch.uint8, device=dev)
    bias = torch.from_numpy(synth.make_layer(5, experts=[]).bias).to(dev)
    T = 1
    buf = LayerBuffers.allocate(sh, T, moe.MOE_PATH_DECODE_F32)
    ws = torch.empty((moe.moe_cache_workspace_bytes(sh, T, slots),), dtype=torch.uint8, device=dev)
    xs = []
    for i in range(warm + steps):
        bits, _ = synth.make_tokens(4, T, batch=1000 + i)
        xs.append(torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16))
    copy_stream = torch.cuda.Stream()
    cache = moe.moe_cache_create(sh, slots, dev_slots, host)
    try:
        def step(i):
            moe.moe_cache_layer_decode(cache, xs[i], w_router, bias, shared, buf.topk_idx, buf.topk_w,
                                       buf.y, buf.y_shared, buf.out, ws, copy_stream=copy_stream)
        for i in range(warm):
            step(i)
        torch.cuda.synchronize()
        h0, m0, b0 = moe.moe_cache_stats(cache)
        t0 = time.perf_counter()
        for i in range(warm, warm + steps):
            step(i)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        h1, m1, b1 = moe.moe_cache_stats(cache)
    finally:
        torch.cuda.synchronize()
        moe.moe_cache_destroy(cache)
    hits, misses, nbytes = h1 - h0, m1 - m0, b1 - b0
    fetch_gbps = nbytes / dt / 1e9
    hit_rate = hits / max(1, hits + misses)
    log(f"expert cache: {slots} slots, {steps / dt:.1f} tokens/s, hit rate {hit_rate:.3f}, "
        f"{misses / steps:.2f} misses/token, host->HBM {fetch_gbps:.1f} GB/s "
        f"(plain pinned copy {h2d:.1f} GB/s)")
    return {
        "value": round(steps / dt, 2),
        "unit": "tokens/s (one layer)",
        "workload": f"1-token decode steps of the d=6144 f=2048 layer through a {slots}-expert HBM "
                    f"cache ({slots * bb / 1e9:.2f} GB), 256 blocks in pinned host memory, Zipf(1.1) "
                    f"router bias, {warm} warm-up steps then {steps} timed",
        "ms_per_step": round(dt * 1e3 / steps, 3),
        "hit_rate": round(hit_rate, 4),
        "misses_per_step": round(misses / steps, 3),
        "roofline": {"bound": "pcie", "kernel": "host->HBM copies of missed experts",
                     "achieved": round(fetch_gbps, 2), "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(fetch_gbps / PCIE_PEAK_GBPS, 4),
                     "plain_pinned_copy_gbps": round(h2d, 2)},
    }


def bench_prefill(args, torch, moe, synth, LayerBuffers, run_layer, sh, experts, shared, w_router, dev,
                  fmt="int4"):
    """2048-token prefill step of the same layer (Zipf router bias); fmt names
    the expert block format of `experts` (int4 gs64 or MXFP4)."""
    L5 = synth.make_layer(5, experts=[])
    bias = torch.from_numpy(L5.bias).to(dev)
    T = 2048
    bits, _ = synth.make_tokens(5, T)
    x = torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    PRE = moe.MOE_PATH_PREFILL_BF16
    buf = LayerBuffers.allocate(sh, T, PRE)
    try:
        run_layer(x, w_router, bias, experts, shared, buf)
        torch.cuda.synchronize()
    except moe.MoeError as e:
        log(f"prefill not measured: {e}")
        return {"status": str(e)}
    stream = torch.cuda.current_stream()
    n = args.prefill_steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for _ in range(3):
        run_layer(x, w_router, bias, experts, shared, buf)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(n):
        moe.moe_route(sh, x, w_router, bias, buf.topk_idx, buf.topk_w, buf.workspace)
        moe.moe_union(sh, T, buf.topk_idx, buf.counts, buf.offsets, buf.perm, buf.inv_perm, buf.active, buf.n_active)
        ev[i][0].record(stream)
        moe.moe_expert_ffn(sh, x, experts, shared, buf.offsets, buf.perm, buf.active, buf.n_active, PRE,
                           buf.y, buf.y_shared, buf.ffn_workspace)
        ev[i][1].record(stream)
        moe.moe_combine(sh, buf.y, buf.y_shared, buf.inv_perm, buf.topk_w, buf.out)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = elapsed * 1e3 / n
    ffn_ms = np.array([s.elapsed_time(e) for s, e in ev])
    flops = 6.0 * sh.d * sh.f * (T * sh.top_k + T)
    tflops = flops / (ffn_ms.mean() * 1e-3) / 1e12
    n_active = int(buf.n_active.item())
    log(f"{fmt} prefill step: {ms:.3f} ms ({T / ms * 1e3:.0f} tokens/s); expert FFN {ffn_ms.mean():.3f} ms "
        f"= {tflops:.0f} TFLOP/s ({n_active} active experts)")
    return {
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "steps": n,
        "dtype": "bf16",
        "workload": "prefill, 2048 tokens, same layer, Zipf(1.1) router bias"
                    + ("" if fmt == "int4" else ", MXFP4 experts (E2M1 + E8M0 per 32)"),
        "active_experts": n_active,
        "roofline": {
            "bound": "mfma",
            "kernel": "moe_expert_ffn (prefill)",
            "achieved": round(tflops, 1),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prefill", fmt),
            "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(float(ffn_ms.mean()) * 1e3, 1),
        },
    }


def counter_workload(args, torch, moe, synth, LayerBuffers, run_layer, dev):
    """The workload of the FETCH_SIZE / WRITE_SIZE counter passes: a plain
    1 GiB device-to-device copy, three times (reads and writes exactly 2^30
    bytes each: the calibration of the counters), then 20 one-token decode
    expert-FFN launches on rotating layer copies, as in the timed run, then
    three 2048-token prefill expert-FFN launches (Zipf-biased routing); then
    the same decode and prefill launches over MXFP4 experts of the same
    geometry."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    L = synth.make_layer(4)
    sh = moe.shape_of(L.shape)
    src = torch.from_numpy(L.experts).to(dev)
    experts = [torch.empty_like(src)]
    moe.moe_pack_experts(sh, L.shape.n_experts, src, experts[0])
    del src
    src = torch.from_numpy(L.shared[None]).to(dev)
    shared = [torch.empty_like(src)[0]]
    moe.moe_pack_experts(sh, 1, src, shared[0])
    del src
    for _ in range(3):
        experts.append(experts[0].clone())
        shared.append(shared[0].clone())
    w_router = torch.from_numpy(L.w_router).to(dev)
    DEC = moe.MOE_PATH_DECODE_F32
    xs, bufs = [], []
    for i in range(4):
        bits, _ = synth.make_tokens(4, 1, batch=i)
        xs.append(torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16))
        bufs.append(LayerBuffers.allocate(sh, 1, DEC))
        run_layer(xs[i], w_router, None, experts[i], shared[i], bufs[i])
    torch.cuda.synchronize()
    for i in range(20):
        b = bufs[i % 4]
        moe.moe_expert_ffn(sh, xs[i % 4], experts[i % 4], shared[i % 4], b.offsets, b.perm,
                           b.active, b.n_active, DEC, b.y, b.y_shared, b.ffn_workspace)
    torch.cuda.synchronize()
    active = [int(b.n_active.item()) + 1 for b in bufs]
    L5 = synth.make_layer(5, experts=[])
    bits, _ = synth.make_tokens(5, 2048)
    x5 = torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    PRE = moe.MOE_PATH_PREFILL_BF16
    pb = LayerBuffers.allocate(sh, 2048, PRE)
    run_layer(x5, w_router, torch.from_numpy(L5.bias).to(dev), experts[0], shared[0], pb)
    for _ in range(3):
        moe.moe_expert_ffn(sh, x5, experts[0], shared[0], pb.offsets, pb.perm, pb.active,
                           pb.n_active, PRE, pb.y, pb.y_shared, pb.ffn_workspace)
    torch.cuda.synchronize()
    del experts, shared
    # the same launches over MXFP4 blocks (same router, so the same grouping)
    Lm = synth.make_layer(4, fmt="mxfp4")
    shm = moe.Shape(sh.d, sh.f, sh.n_experts, sh.top_k, 32, sh.f_shared)
    src = torch.from_numpy(Lm.experts).to(dev)
    mx = [torch.empty_like(src)]
    moe.moe_pack_experts(shm, Lm.shape.n_experts, src, mx[0])
    del src
    src = torch.from_numpy(Lm.shared[None]).to(dev)
    mxs = [torch.empty_like(src)[0]]
    moe.moe_pack_experts(shm, 1, src, mxs[0])
    del src, Lm
    for _ in range(3):
        mx.append(mx[0].clone())
        mxs.append(mxs[0].clone())
    torch.cuda.synchronize()
    for i in range(20):
        b = bufs[i % 4]
        moe.moe_expert_ffn(shm, xs[i % 4], mx[i % 4], mxs[i % 4], b.offsets, b.perm, b.active,
                           b.n_active, DEC, b.y, b.y_shared, b.ffn_workspace)
    for _ in range(3):
        moe.moe_expert_ffn(shm, x5, mx[0], mxs[0], pb.offsets, pb.perm, pb.active, pb.n_active,
                           PRE, pb.y, pb.y_shared, pb.ffn_workspace)
    torch.cuda.synchronize()
    log(f"counter workload done: copy 3 x {n} B; 20 decode FFN launches of {active} expert blocks; "
        f"3 prefill FFN launches ({int(pb.n_active.item())} active experts); the same over "
        f"MXFP4 blocks")
    return 0


def load_traffic(which="decode", fmt="int4"):
    """HBM bytes per expert-FFN launch (decode or prefill; int4 or MXFP4
    blocks) from the committed counter summary, or None when that path's
    kernel source has changed since the counters were taken (its SHA-256 is
    recorded with them)."""
    import hashlib
    suffix = "" if fmt == "int4" else "_" + fmt
    path = os.path.join(ROOT, "profiles", f"{which}_ffn_traffic{suffix}.json")
    src = os.path.join(ROOT, "int4_routed_expert_logits_amd", "csrc", f"ffn_{which}.hip")
    try:
        with open(path) as fh:
            rec = json.load(fh)
        with open(src, "rb") as fh:
            digest = hashlib.sha256(fh.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != digest:
        return None
    return rec.get("bytes_per_launch")


def cpu_info():
    """Host CPU as the oracle sees it: logical CPUs this process may use, all
    logical CPUs, and the model name."""
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, os.cpu_count(), model


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return None


def cpu_baseline(L, bb):
    """The float64 oracle, as it stands, on the host cores.
    Decode (the headline unit): whole 1-token decode steps of the same layer
    (routing, grouping, 8 routed + 1 shared expert, combine), repeated until
    ~10 s of CPU work.  Prefill: the 2048-token Zipf batch's routing and
    grouping in full, then the oracle's expert FFN on a sample of 16 of its
    active experts spread over the row-count range (decode the block, SwiGLU
    over the expert's rows); the whole batch's time is extrapolated as
    (active experts) x (mean block decode time) + (all rows) x (SwiGLU time
    per row of the sample)."""
    import oracle
    import synth
    usable, logical, model = cpu_info()
    threads = blas_threads() or usable
    sh = L.shape
    reps = 0
    elapsed = 0.0
    blocks = 0
    while elapsed < 10.0 and reps < 8:
        _, xf = synth.make_tokens(4, 1, batch=100 + reps)
        t = time.perf_counter()
        res = oracle.moe_layer(xf, L.w_router, None, L.experts, L.shared, sh.d, sh.f,
                               sh.n_experts, sh.top_k)
        elapsed += time.perf_counter() - t
        blocks += int(res["n_active"][0]) + 1
        reps += 1
    gbps = blocks * bb / elapsed / 1e9
    log(f"cpu oracle: {reps} decode steps in {elapsed:.1f}s = {gbps:.4f} GB/s ({threads} BLAS "
        f"threads, {usable} usable CPUs, {model})")
    # prefill sample
    bias = synth.make_layer(5, experts=[]).bias
    _, xf = synth.make_tokens(5, 2048)
    t = time.perf_counter()
    idx, w, _ = oracle.route(xf, L.w_router, bias, sh.top_k)
    counts, offsets, perm, inv, active, n_active = oracle.batch_union(idx, sh.n_experts)
    t_route = time.perf_counter() - t
    act = [int(e) for e in active[: int(n_active[0])]]
    order = sorted(act, key=lambda e: int(counts[e]))
    pick = [order[i * (len(order) - 1) // 15] for i in range(16)]
    t_dec = t_mm = 0.0
    rows = 0
    x64 = np.asarray(xf, dtype=np.float64)
    for e in pick:
        t0 = time.perf_counter()
        wg, wu, wd = oracle.expert_weights(L.experts[e], sh.d, sh.f)
        t1 = time.perf_counter()
        toks = np.asarray(perm[offsets[e]:offsets[e + 1]], dtype=np.int64) // sh.top_k
        oracle.swiglu(x64[toks], wg, wu, wd)
        t2 = time.perf_counter()
        t_dec += t1 - t0
        t_mm += t2 - t1
        rows += len(toks)
        del wg, wu, wd
    all_rows = 2048 * sh.top_k + 2048  # routed rows + the shared expert's
    est = t_route + (len(act) + 1) * t_dec / len(pick) + all_rows * t_mm / rows
    log(f"cpu oracle prefill: {len(pick)} of {len(act)} experts ({rows} rows) in "
        f"{t_dec + t_mm:.1f}s; whole 2048-token batch extrapolated to {est:.0f}s = "
        f"{2048 / est:.1f} tokens/s")
    return {"value": round(gbps, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} one-token decode steps of the same layer ({blocks} expert blocks), "
                      f"float64 numpy oracle, {elapsed:.1f} s",
            "cpu_model": model, "usable_cpus": usable, "logical_cpus": logical,
            "cores_note": "cores = threads of numpy's BLAS pool (the oracle's matrix products); "
                          "its element-wise decoding runs on one thread",
            "prefill": {"value": round(2048 / est, 2), "unit": "tokens/s", "extrapolated": True,
                        "seconds_estimated": round(est, 1),
                        "sample": f"routing and grouping of the 2048-token Zipf batch in full "
                                  f"({t_route:.1f} s); the expert FFN of {len(pick)} of its "
                                  f"{len(act)} active experts ({rows} rows) in "
                                  f"{t_dec + t_mm:.1f} s, extrapolated by block count and rows"}}


if __name__ == "__main__":
    sys.exit(main())
