"""Benchmark of the MI355X int8 convrot linear layer.

One step = one int8_compute forward of the Z-Image-like attention projection
(x bf16 [4608, 3840] -> y bf16 [4608, 3840], W int8 [3840, 3840], g = 256,
seeded Hadamard-sign rotation): convrot_linear_int8, i.e. the fused
rotate + absmax + quantize kernel(s) followed by the int8 MFMA GEMM.

value = 2*M*N*K / (time per step), in TOPS (int8 ops).

Also measured, each with HIP events on the stream its kernels run on:
  gemm       - the int8 GEMM kernel alone: TOPS and fraction of the 5.0 POP/s
               int8 dense MFMA peak (the "roofline" object);
  act_quant  - activation rotate + quantize: algorithmic 3 B per element +
               4 B per token, GB/s and fraction of 8 TB/s;
  dequant    - weight dequant + derotate: 1 B read + 2 B written per element
               (+ 4 B scale), GB/s and fraction of 8 TB/s.
Inputs are rotated over enough buffers that the bytes touched between two uses
of one buffer exceed twice the 256 MB MALL, so HBM, not cache, is measured.

cpu_baseline: the CPU oracle (numpy/float64, as it stands) timed on the
host's cores over a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
MALL_BYTES = 256 << 20
HOLD_MS = 20.0        # minimum GPU-side hold before a launch-bound timed batch
HOLD_CYCLES_PER_MS = 2.4e6  # torch.cuda._sleep counts shader clocks (~2.4 GHz)
WARM_GPU_MS = 20.0    # untimed GPU work between the hold and the first event
MIN_WARM, MAX_WARM = 2, 4000
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_zimage_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "int8_gemm_amd", "csrc", "gemm.hip")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks settle over the first ~10 ms of load: the default
    # warm-up covers that, and the timed region (~50 ms) averages out noise
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample (10-30 s)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline line: one JSON line per workload config "
                         "(GEMM, linear, act-quant and dequant, HIP-event means)")
    ap.add_argument("--warm-ms", type=float, default=WARM_GPU_MS,
                    help="untimed GPU work before each timed batch (clock ramp); counter "
                         "passes, which time nothing, may set it to 0")
    return ap.parse_args()


def _source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(n_launch_units: float):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    if it was taken on the current GEMM source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != _source_hash(GEMM_SOURCE):
        return None
    return t.get("hbm_bytes_per_launch")


def _probe_ms(fn, stream):
    """(GPU ms per launch, host ms per call) of `fn` from a short batch of
    ~2 ms. The events measure the kernel itself when the host enqueues faster
    than the GPU runs it, else (a launch-bound call) about the host's rate."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn(0)
    e1.record(stream)
    torch.cuda.synchronize()
    n = int(min(100, max(1, 2.0 / max(e0.elapsed_time(e1), 1e-3))))
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    host = (time.perf_counter() - t0) * 1e3 / n
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, host


def _events_time(fn, reps, stream):
    """GPU duration per launch from HIP events recorded on `stream`.

    Every timed batch follows WARM_GPU_MS of untimed launches of the same
    call, so caches and clocks are in their steady state. A call whose kernel
    runs less than twice as long as the host takes to issue it would leave
    launch gaps: for those the stream is first held by a GPU-side sleep long
    enough for the host to enqueue the warm-up and the batch (the host's
    per-call cost is measured first); the clocks fall during the hold, and
    the warm-up brings them back. Longer kernels need no hold: the host gets
    ahead of the GPU on its own. Returns (mean, min, median) in ms: the mean
    over a batch of `reps` back-to-back launches between two events
    (per-event overhead amortised, as a kernel trace sees it; the median of 3
    such batches), min and median over launches bracketed one by one."""
    import torch
    kern_ms, host_ms = _probe_ms(fn, stream)
    warm = int(min(MAX_WARM, max(MIN_WARM, math.ceil(WARM_GPU_MS / max(kern_ms, 1e-4)))))

    def held_warm(margin):
        # margin: host cost per call relative to the probe's (event records add to it)
        if kern_ms < 2.0 * margin * host_ms:
            hold_ms = max(HOLD_MS, 1.5 * margin * (warm + reps) * host_ms)
            with torch.cuda.stream(stream):
                torch.cuda._sleep(int(hold_ms * HOLD_CYCLES_PER_MS))
        for i in range(warm):
            fn(i)

    means = []
    for _ in range(3):
        held_warm(1.0)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(reps):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        means.append(t0.elapsed_time(t1) / reps)
    mean = sorted(means)[1]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    held_warm(2.0)
    for i in range(reps):
        starts[i].record(stream)
        fn(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return mean, ms[0], ms[len(ms) // 2]


def _cpu_baseline(layer, g, seed, target_s):
    """The oracle's int8 forward (rotate + quantize + int32 GEMM + epilogue)
    over row chunks of the same workload until ~target_s seconds pass."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    import oracle
    xb, wb = layer.x(), layer.w()
    wq, s_w = oracle.quantize_weights(wb, g, seed)
    chunk = 512
    rows_done = 0
    t0 = time.perf_counter()
    while True:
        r0 = rows_done % layer.m
        oracle.linear_int8(np.ascontiguousarray(xb[r0:r0 + chunk]), wq, s_w, g, seed)
        rows_done += min(chunk, layer.m - r0)
        el = time.perf_counter() - t0
        if el >= target_s or el > 30.0:
            break
    tops = 2.0 * rows_done * layer.n * layer.k / el / 1e12
    return {"value": round(tops, 6), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows_done} token rows (chunks of {chunk}) of the {layer.m}x{layer.n}x"
                      f"{layer.k} layer through oracle.linear_int8 (numpy float64 BLAS), "
                      f"{el:.1f} s"}


def _all_configs(reps: int):
    """One JSON line per workload config: the GEMM (default tile), the whole
    int8 forward with the default workspace, the activation quantization and
    the dequant + derotate, each as the HIP-event mean of back-to-back
    launches; input and output buffers rotated so that the data touched
    between two uses of a buffer exceeds twice the 256 MB MALL (footprints of
    at least 512 MB need no rotation)."""
    import numpy as np
    import torch

    import int8_gemm_amd as cr
    import synth

    cr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    seed = synth.ROT_SEED
    cases = [(synth.TINY, 256), (synth.ZIMAGE_ATTN, 256), (synth.FLUX_MLP_UP, 256),
             (synth.FLUX_MLP_DOWN, 256), (synth.WAN_FFN_UP, 256), (synth.WAN_FFN_DOWN, 256)] + \
        [(synth.QKV_SWEEP, g) for g in synth.GROUP_SIZES]

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def copies(t, footprint):
        n = 1 if footprint >= 2 * MALL_BYTES else max(2, math.ceil(2 * MALL_BYTES / footprint) + 1)
        return [t] + [t.clone() for _ in range(n - 1)]

    for layer, g in cases:
        print(f"[bench] config {layer.name} g={g}", file=sys.stderr, flush=True)
        m, n, k = layer.m, layer.n, layer.k
        x0 = to_dev(layer.x())
        wq, s_w = cr.convrot_quantize_weights(to_dev(layer.w()), g, seed)
        xs = copies(x0, 3 * m * k)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        sx = torch.empty(m, dtype=torch.float32, device=dev)
        cr.convrot_quantize_activations(x0, g, seed, xq=xq, s_x=sx)
        ys = copies(torch.empty((m, n), dtype=torch.bfloat16, device=dev), 2 * m * n)
        ws = torch.empty(cr.convrot_linear_int8_workspace_size(m, n, k), dtype=torch.uint8,
                         device=dev)
        act_ms, _, _ = _events_time(lambda i: cr.convrot_quantize_activations(
            xs[i % len(xs)], g, seed, xq=xq, s_x=sx), reps, stream)
        gemm_ms, _, _ = _events_time(lambda i: cr.convrot_gemm_int8(
            xq, sx, wq, s_w, y=ys[i % len(ys)]), reps, stream)
        lin_ms, _, _ = _events_time(lambda i: cr.convrot_linear_int8(
            xs[i % len(xs)], wq, s_w, g, seed, workspace=ws, out=ys[i % len(ys)]), reps, stream)
        del xs, ys, ws, xq
        wqs = copies(wq, 3 * n * k)
        outs = copies(torch.empty((n, k), dtype=torch.bfloat16, device=dev), 3 * n * k)
        deq_ms, _, _ = _events_time(lambda i: cr.convrot_dequant_derotate(
            wqs[i % len(wqs)], s_w, g, seed, out=outs[i % len(outs)]), reps, stream)
        del wqs, outs
        torch.cuda.synchronize()
        ops = 2.0 * m * n * k
        act_b, deq_b = 3.0 * m * k + 4.0 * m, 3.0 * n * k + 4.0
        print(json.dumps({
            "config": layer.name, "m": m, "n": n, "k": k, "g": g,
            "gemm_TOPS": round(ops / (gemm_ms * 1e-3) / 1e12, 1),
            "gemm_frac_peak": round(ops / (gemm_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "linear_TOPS": round(ops / (lin_ms * 1e-3) / 1e12, 1),
            "act_quant_GB/s": round(act_b / (act_ms * 1e-3) / 1e9, 1),
            "act_quant_frac_hbm": round(act_b / (act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "dequant_GB/s": round(deq_b / (deq_ms * 1e-3) / 1e9, 1),
            "dequant_frac_hbm": round(deq_b / (deq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "us": {"gemm": round(gemm_ms * 1e3, 2), "linear": round(lin_ms * 1e3, 2),
                   "act_quant": round(act_ms * 1e3, 2), "dequant": round(deq_ms * 1e3, 2)}}),
            flush=True)


def main():
    global WARM_GPU_MS
    args = _parse()
    WARM_GPU_MS = max(0.0, args.warm_ms)
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the layer "
              "shards by tokens or output features without any communication, so a "
              "multi-GPU figure is the one-GPU figure per GPU", file=sys.stderr)
        sys.exit(2)
    if args.all_configs:
        _all_configs(min(max(args.steps, 10), 50))
        return

    import numpy as np
    import torch

    import int8_gemm_amd as cr
    import synth

    cr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layer, g, seed = synth.ZIMAGE_ATTN, 256, synth.ROT_SEED
    m, n, k = layer.m, layer.n, layer.k
    print(f"[bench] workload {layer.name} g={g}: generating inputs", file=sys.stderr, flush=True)
    xb, wb = layer.x(), layer.w()

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x0, w = to_dev(xb), to_dev(wb)
    wq, s_w = cr.convrot_quantize_weights(w, g, seed)
    stream = torch.cuda.current_stream(dev)

    # rotating buffer sets (> 2 x MALL between reuses)
    x_bytes = m * k * 2
    nrot_x = max(2, math.ceil(2 * MALL_BYTES / x_bytes) + 1)
    xs = [x0] + [x0.clone() for _ in range(nrot_x - 1)]
    ws = torch.empty(cr.convrot_linear_int8_workspace_size(m, n, k), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)

    def step(i):
        cr.convrot_linear_int8(xs[i % nrot_x], wq, s_w, g, seed, workspace=ws, out=y)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    ops = 2.0 * m * n * k
    value = ops / (ms_step * 1e-3) / 1e12

    # ---- per-kernel timings (HIP events on the launch stream) ----
    reps = min(max(args.steps, 10), 200)
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    sx = torch.empty(m, dtype=torch.float32, device=dev)
    cr.convrot_quantize_activations(x0, g, seed, xq=xq, s_x=sx)
    act_ms, act_min, _ = _events_time(
        lambda i: cr.convrot_quantize_activations(xs[i % nrot_x], g, seed, xq=xq, s_x=sx),
        reps, stream)
    gemm_ms, gemm_min, gemm_med = _events_time(
        lambda i: cr.convrot_gemm_int8(xq, sx, wq, s_w, y=y), reps, stream)
    tiles = {}
    for t in (128, 192, 256, 384):
        t_ms, _, _ = _events_time(
            lambda i: cr.convrot_gemm_int8(xq, sx, wq, s_w, y=y, tile=t), reps, stream)
        tiles[str(t)] = round(2.0 * m * n * k / (t_ms * 1e-3) / 1e12, 1)
    wset = n * k * 3
    nrot_w = max(2, math.ceil(2 * MALL_BYTES / wset) + 1)
    wqs = [wq] + [wq.clone() for _ in range(nrot_w - 1)]
    outs = [torch.empty((n, k), dtype=torch.bfloat16, device=dev) for _ in range(nrot_w)]
    deq_ms, deq_min, _ = _events_time(
        lambda i: cr.convrot_dequant_derotate(wqs[i % nrot_w], s_w, g, seed,
                                              out=outs[i % nrot_w]), reps, stream)
    torch.cuda.synchronize()

    # ---- per-output-channel weight scales: the same layer, one fp32 scale per
    # weight row; the int8 forward, its GEMM and the dequant ----
    wq_pc, sw_pc = cr.convrot_quantize_weights_per_channel(w, g, seed)
    pc_lin_ms, _, _ = _events_time(
        lambda i: cr.convrot_linear_int8_per_channel(xs[i % nrot_x], wq_pc, sw_pc, g, seed,
                                                     workspace=ws, out=y), reps, stream)
    pc_gemm_ms, _, _ = _events_time(
        lambda i: cr.convrot_gemm_int8_per_channel(xq, sx, wq_pc, sw_pc, y=y), reps, stream)
    wqs_pc = [wq_pc] + [wq_pc.clone() for _ in range(nrot_w - 1)]
    pc_deq_ms, _, _ = _events_time(
        lambda i: cr.convrot_dequant_derotate_per_channel(wqs_pc[i % nrot_w], sw_pc, g, seed,
                                                          out=outs[i % nrot_w]), reps, stream)
    torch.cuda.synchronize()
    del wqs, outs, wqs_pc, wq_pc

    # ---- FP16 activations and outputs: the same layer with x, y in half ----
    xh0 = torch.from_numpy(layer.x(fmt="f16").view(np.int16)).view(torch.float16).to(dev)
    xhs = [xh0] + [xh0.clone() for _ in range(nrot_x - 1)]
    yh = torch.empty((m, n), dtype=torch.float16, device=dev)
    h_lin_ms, _, _ = _events_time(
        lambda i: cr.convrot_linear_int8_ex(xhs[i % nrot_x], wq, s_w, g, seed, workspace=ws,
                                            out=yh), reps, stream)
    h_act_ms, _, _ = _events_time(
        lambda i: cr.convrot_quantize_activations_ex(xhs[i % nrot_x], g, seed, xq=xq, s_x=sx),
        reps, stream)
    torch.cuda.synchronize()
    del xhs, xh0, yh

    # ---- dequant over the 60-layer stack: 60 + 60 distinct int8 buffers of
    # the two stack shapes, one dequant each per pass, outputs rotated over 4 ----
    stack = []
    for lay in (synth.STACK_SQUARE, synth.STACK_WIDE):
        wq_l, sw_l = cr.convrot_quantize_weights(to_dev(lay.w()), g, seed)
        copies = [wq_l.clone() for _ in range(synth.STACK_LAYERS)]
        del wq_l
        outs_l = [torch.empty((lay.n, lay.k), dtype=torch.bfloat16, device=dev)
                  for _ in range(4)]
        stack.append((copies, sw_l, outs_l))

    def stack_pass(i):
        for layer_i in range(synth.STACK_LAYERS):
            for copies, sw_l, outs_l in stack:
                cr.convrot_dequant_derotate(copies[layer_i], sw_l, g, seed,
                                            out=outs_l[layer_i % 4])

    stack_ms, stack_min, _ = _events_time(stack_pass, 3, stream)
    stack_bytes = float(sum(3 * c[0].numel() * len(c) + 4 * len(c) for c, _, _ in stack))

    # ---- the same 60 + 60 stack streamed from pinned host memory: 4608
    # tokens through every layer, each layer's int8 weight copied to the GPU
    # on the streamer's copy stream while earlier layers compute ----
    print("[bench] streamed stack", file=sys.stderr, flush=True)
    sm_tok = layer.m
    xs_k = to_dev(synth.activations(sm_tok, synth.STACK_SQUARE.k, 505))
    host_layers, dev_layers = [], []
    for layer_i in range(synth.STACK_LAYERS):
        for copies, sw_l, _ in stack:
            host_layers.append((copies[layer_i].cpu().pin_memory(), sw_l))
            dev_layers.append((copies[layer_i], sw_l))
    stream_bytes = float(sum(w.numel() for w, _ in host_layers))
    ys = {n_: torch.empty((sm_tok, n_), dtype=torch.bfloat16, device=dev)
          for n_ in {w.shape[0] for w, _ in host_layers}}
    ws_s = torch.empty(max(cr.convrot_linear_int8_workspace_size(sm_tok, n_, xs_k.shape[1])
                           for n_ in ys), dtype=torch.uint8, device=dev)
    slot_bytes = max(w.numel() for w, _ in host_layers)
    streamer = cr.Streamer(slot_bytes, 2)

    def streamed_pass(i):
        for wh, sw_l in host_layers:
            streamer.linear(xs_k, wh, sw_l, g, seed, workspace=ws_s, out=ys[wh.shape[0]])

    def resident_pass(i):
        for wd, sw_l in dev_layers:
            cr.convrot_linear_int8(xs_k, wd, sw_l, g, seed, workspace=ws_s, out=ys[wd.shape[0]])

    staging = torch.empty(slot_bytes, dtype=torch.int8, device=dev)

    def copy_pass(i):
        for wh, _ in host_layers:
            staging[:wh.numel()].copy_(wh.view(-1), non_blocking=True)

    streamed_pass(0)
    torch.cuda.synchronize()
    str_ms, _, _ = _events_time(streamed_pass, 2, stream)
    res_ms, _, _ = _events_time(resident_pass, 2, stream)
    cpy_ms, _, _ = _events_time(copy_pass, 2, stream)
    streamer.close()
    stack_ops = float(sum(2.0 * sm_tok * w.shape[0] * w.shape[1] for w, _ in host_layers))
    del stack, host_layers, dev_layers, ys, ws_s, staging, xs_k
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    act_bytes = 3.0 * m * k + 4.0 * m
    deq_bytes = 3.0 * n * k + 4.0
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    act_gbs = act_bytes / (act_ms * 1e-3) / 1e9
    deq_gbs = deq_bytes / (deq_ms * 1e-3) / 1e9
    traffic = _traffic(1)

    result = {
        "metric": "int8 convrot linear TOPS (+% int8 MFMA peak); dequant/act-quant GB/s "
                  "(+% HBM)",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"{layer.name}: x bf16 [{m},{k}] (0.5% outlier channels x30), "
                               f"W int8 [{n},{k}] (1% outlier columns x10), g={g}, "
                               "R = Walsh-Hadamard x seeded signs",
                   "m": m, "n": n, "k": k, "g": g, "rot_seed": seed,
                   "x_buffers_rotated": nrot_x},
        "roofline": {"bound": "mfma", "kernel": "gemm_i8_kernel",
                     "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                     "traffic": traffic,
                     "avg_ms": round(gemm_ms, 5), "min_ms": round(gemm_min, 5),
                     "tops_by_forced_tile": tiles},
        "act_quant": {"GB/s": round(act_gbs, 1), "frac_hbm": round(act_gbs / PEAK_HBM_GBS, 4),
                      "avg_ms": round(act_ms, 5), "min_ms": round(act_min, 5),
                      "bytes": act_bytes},
        "dequant": {"GB/s": round(deq_gbs, 1), "frac_hbm": round(deq_gbs / PEAK_HBM_GBS, 4),
                    "avg_ms": round(deq_ms, 5), "min_ms": round(deq_min, 5),
                    "bytes": deq_bytes, "buffers_rotated": nrot_w},
        "dequant_stack": {"layers": 2 * synth.STACK_LAYERS,
                          "GB/s": round(stack_bytes / (stack_ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(stack_bytes / (stack_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "ms_per_pass": round(stack_ms, 4), "bytes": stack_bytes},
        "linear_tops_frac_peak": round(value / PEAK_INT8_TOPS, 4),
        "streamed_stack": {
            "layers": 2 * synth.STACK_LAYERS, "tokens": sm_tok,
            "int8_bytes_per_pass": stream_bytes,
            "ms_per_pass": round(str_ms, 3),
            "h2d_GB/s": round(stream_bytes / (str_ms * 1e-3) / 1e9, 1),
            "copy_only_ms": round(cpy_ms, 3),
            "copy_only_GB/s": round(stream_bytes / (cpy_ms * 1e-3) / 1e9, 1),
            "frac_of_copy_only": round(cpy_ms / str_ms, 4),
            "resident_ms_per_pass": round(res_ms, 3),
            "resident_TOPS": round(stack_ops / (res_ms * 1e-3) / 1e12, 1),
            "streamed_TOPS": round(stack_ops / (str_ms * 1e-3) / 1e12, 1)},
        "per_channel": {
            "linear_TOPS": round(ops / (pc_lin_ms * 1e-3) / 1e12, 1),
            "gemm_TOPS": round(ops / (pc_gemm_ms * 1e-3) / 1e12, 1),
            "gemm_frac_peak": round(ops / (pc_gemm_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "dequant_GB/s": round((3.0 * n * k + 4.0 * n) / (pc_deq_ms * 1e-3) / 1e9, 1),
            "dequant_frac_hbm": round((3.0 * n * k + 4.0 * n) / (pc_deq_ms * 1e-3) / 1e9
                                      / PEAK_HBM_GBS, 4),
            "linear_avg_ms": round(pc_lin_ms, 5), "gemm_avg_ms": round(pc_gemm_ms, 5),
            "dequant_avg_ms": round(pc_deq_ms, 5)},
        "f16": {
            "linear_TOPS": round(ops / (h_lin_ms * 1e-3) / 1e12, 1),
            "act_quant_GB/s": round(act_bytes / (h_act_ms * 1e-3) / 1e9, 1),
            "act_quant_frac_hbm": round(act_bytes / (h_act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "linear_avg_ms": round(h_lin_ms, 5), "act_quant_avg_ms": round(h_act_ms, 5)},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = _cpu_baseline(layer, g, seed, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
