"""Benchmark of the MI355X int8 convrot linear layer.

One step = one int8_compute forward of the Wan-like FFN pair on video tokens
(the largest single-GPU workload): x1 bf16 [32760, 5120] -> y1 [32760, 13824]
through W1 int8 [13824, 5120], then x2 bf16 [32760, 13824] -> y2 [32760, 5120]
through W2 int8 [5120, 13824], g = 256, seeded Hadamard-sign rotation. Each
is a convrot_linear_int8 call with the default workspace (token slices of at
most 2N rows): the fused rotate + absmax + quantize kernel(s), then the int8
MFMA GEMM with its scaling epilogue.

value = 2*M*N*K of both legs / (time per step), in TOPS (int8 ops).

Also measured, each with HIP events on the stream its kernels run on:
  roofline   - the int8 GEMM of the up projection (32760 x 13824 x 5120, one
               launch): TOPS against the 5.0 POP/s int8 dense MFMA peak, and
               against the peak at the shader clock sampled while it runs;
  legs       - each linear alone, its GEMM, activation rotate + quantize
               (2 B read + 1 B written per element + 4 B per token) and
               dequant + derotate (1 B read + 2 B written per element + 4 B)
               as GB/s and fraction of 8 TB/s;
  zimage_attn, per_channel, f16, dequant_stack, streamed_stack - the other
               workload shapes and paths;
  copy_ceiling - a plain 1 GiB device-to-device copy (read + write bytes).
Buffers whose footprint is below twice the 256 MB MALL are rotated over
copies, so HBM, not cache, is measured.

cpu_baseline: the CPU oracle (numpy/float64, as it stands) timed on the host's
cores over a bounded sample of the same workload, per stage.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOPS
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
NUM_CUS = 256
INT8_OPS_PER_CLK_PER_CU = 8192  # v_mfma_i32_32x32x32_i8: 4 SIMDs
MALL_BYTES = 256 << 20
HOLD_MS = 20.0        # minimum GPU-side hold before a launch-bound timed batch
HOLD_CYCLES_PER_MS = 2.4e6  # torch.cuda._sleep counts shader clocks (~2.4 GHz)
WARM_GPU_MS = 20.0    # untimed GPU work between the hold and the first event
STEP_WARM_MS = 60.0   # untimed steps before the headline's timed steps
MIN_WARM, MAX_WARM = 2, 4000
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_wan_ffn_up_traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "int8_gemm_amd", "csrc", "gemm.hip")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample (10-30 s)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy three times (counter calibration)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline line: one JSON line per workload config "
                         "(GEMM, linear, act-quant and dequant, HIP-event means)")
    ap.add_argument("--warm-ms", type=float, default=WARM_GPU_MS,
                    help="untimed GPU work before each timed batch (clock ramp); counter "
                         "passes, which time nothing, may set it to 0")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the FFN pair, its legs and the roofline GEMM (profiling runs)")
    ap.add_argument("--leg", choices=("act_quant", "dequant", "gemm", "linear", "vendor_gemm"),
                    help="instead of the headline line: time one leg of one workload "
                         "(--config, --g) over --steps launches (counter and trace runs)")
    ap.add_argument("--config", default="wan-ffn-up",
                    help="workload of --leg: " + ", ".join(_CONFIG_NAMES))
    ap.add_argument("--g", type=int, default=256, help="group size of --leg")
    return ap.parse_args()


_CONFIG_NAMES = ("tiny", "zimage-attn", "flux-mlp-up", "flux-mlp-down", "wan-ffn-up",
                 "wan-ffn-down", "fused-qkv")


def _one_leg(args):
    """One leg of one workload, `args.steps` launches after a warm-up, with the
    buffers rotated past the MALL; prints one JSON line (HIP-event mean)."""
    import numpy as np
    import torch

    import int8_gemm_amd as cr
    import synth
    layers = dict(zip(_CONFIG_NAMES, synth.ALL_LAYERS))
    layer, g, seed = layers[args.config], args.g, synth.ROT_SEED
    m, n, k = layer.m, layer.n, layer.k
    cr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    wq, s_w = cr.convrot_quantize_weights(to_dev(layer.w()), g, seed)
    x0 = to_dev(layer.x())
    if args.leg == "dequant":
        wqs = _copies(wq, 3 * n * k)
        outs = _copies(torch.empty((n, k), dtype=torch.bfloat16, device=dev), 3 * n * k)
        fn = lambda i: cr.convrot_dequant_derotate(wqs[i % len(wqs)], s_w, g, seed,  # noqa: E731
                                                   out=outs[i % len(outs)])
        units, unit = 3.0 * n * k + 4.0, "GB/s"
    else:
        xs = _copies(x0, 3 * m * k)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        sx = torch.empty(m, dtype=torch.float32, device=dev)
        cr.convrot_quantize_activations(x0, g, seed, xq=xq, s_x=sx)
        ys = _copies(torch.empty((m, n), dtype=torch.bfloat16, device=dev), 2 * m * n)
        ws = torch.empty(cr.convrot_linear_int8_workspace_size(m, n, k), dtype=torch.uint8,
                         device=dev)
        if args.leg == "act_quant":
            fn = lambda i: cr.convrot_quantize_activations(  # noqa: E731
                xs[i % len(xs)], g, seed, xq=xq, s_x=sx)
            units, unit = 3.0 * m * k + 4.0 * m, "GB/s"
        elif args.leg == "gemm":
            fn = lambda i: cr.convrot_gemm_int8(xq, sx, wq, s_w, y=ys[i % len(ys)])  # noqa: E731
            units, unit = 2.0 * m * n * k, "TOPS"
        elif args.leg == "vendor_gemm":
            # reference point only: the platform's int8 GEMM (torch._int_mm, int32
            # out, no scaling epilogue) on the same operands; not this library
            wt = wq.t()
            fn = lambda i: torch._int_mm(xq, wt)  # noqa: E731
            units, unit = 2.0 * m * n * k, "TOPS"
        else:
            fn = lambda i: cr.convrot_linear_int8(  # noqa: E731
                xs[i % len(xs)], wq, s_w, g, seed, workspace=ws, out=ys[i % len(ys)])
            units, unit = 2.0 * m * n * k, "TOPS"
    ms = _events_time(fn, max(1, args.steps), stream, batches=1)
    rate = units / (ms * 1e-3) / (1e12 if unit == "TOPS" else 1e9)
    print(json.dumps({"leg": args.leg, "config": layer.name, "g": g, "us": round(ms * 1e3, 2),
                      unit: round(rate, 1)}), flush=True)


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
    v = t.get("hbm_bytes_per_launch")
    return None if v is None else v * n_launch_units


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

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


def _events_time(fn, reps, stream, batches=3):
    """GPU ms per launch of `fn` from HIP events recorded on `stream`: the
    median over `batches` batches of `reps` back-to-back launches, each batch
    bracketed by one event pair (per-event overhead amortised, as a kernel
    trace sees it).

    Every batch follows WARM_GPU_MS of untimed launches of the same call, so
    caches and clocks are in their steady state. A call whose kernel runs less
    than twice as long as the host takes to issue it would leave launch gaps:
    for those the stream is first held by a GPU-side sleep long enough for the
    host to enqueue the warm-up and the batch (the host's per-call cost is
    measured first); the clocks fall during the hold, and the warm-up brings
    them back. Longer kernels need no hold: the host gets ahead of the GPU on
    its own."""
    import torch
    kern_ms, host_ms = _probe_ms(fn, stream)
    warm = int(min(MAX_WARM, max(MIN_WARM, math.ceil(WARM_GPU_MS / max(kern_ms, 1e-4)))))
    means = []
    for _ in range(batches):
        if kern_ms < 2.0 * host_ms:
            hold_ms = max(HOLD_MS, 1.5 * (warm + reps) * host_ms)
            with torch.cuda.stream(stream):
                torch.cuda._sleep(int(hold_ms * HOLD_CYCLES_PER_MS))
        for i in range(warm):
            fn(i)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(reps):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        means.append(t0.elapsed_time(t1) / reps)
    return sorted(means)[len(means) // 2]


class ClockSampler:
    """Shader clock (MHz, mean over the XCDs) and socket power (W) sampled
    through amdsmi from a background thread while GPU work runs. The
    firmware refreshes the figures every few tens of ms, on some boxes far
    more rarely: a reading equal to the one before it is a repeat of a
    stale figure and is dropped; so are readings taken before `settle_s`
    (the clocks ramp up under load)."""

    def __init__(self, settle_s=0.5, period_s=0.02):
        self.settle_s, self.period_s = settle_s, period_s
        self.samples, self.error = [], None
        self._last, self.reads = None, 0
        self._stop = threading.Event()
        self._handle = None
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if bus is None or int(bdf.split(":")[1], 16) == bus:
                    self._handle = h
                    break
            if self._handle is None:
                self.error = "no amdsmi handle matches the device's PCI bus"
            self._amdsmi = amdsmi
        except Exception as e:  # noqa: BLE001 - amdsmi missing or not permitted
            self.error = f"amdsmi unavailable: {e!r}"[:200]

    def _run(self):
        t0 = time.perf_counter()
        while not self._stop.is_set():
            t = time.perf_counter() - t0
            try:
                m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int)]
                clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
                pw = m.get("current_socket_power")
                pw = pw if isinstance(pw, (int, float)) else None
                if isinstance(clk, (int, float)):
                    fresh = self._last is None or (clk, pw) != self._last
                    self._last = (clk, pw)
                    self.reads += 1
                    if t >= self.settle_s and fresh:
                        self.samples.append((clk, pw))
            except Exception as e:  # noqa: BLE001
                self.error = f"amdsmi read failed: {e!r}"[:200]
                return
            self._stop.wait(self.period_s)

    def run_during(self, fn):
        if self._handle is None:
            fn()
            return
        th = threading.Thread(target=self._run, daemon=True)
        th.start()
        try:
            fn()
        finally:
            self._stop.set()
            th.join()

    def summary(self):
        if not self.samples:
            return {"sclk_MHz": None, "socket_power_W": None, "samples": 0,
                    "note": self.error or "no sample after the settle time"}
        clks = sorted(c for c, _ in self.samples)
        pws = sorted(p for _, p in self.samples if p is not None)
        return {"sclk_MHz": round(clks[len(clks) // 2], 1),
                "sclk_MHz_range": [round(clks[0], 1), round(clks[-1], 1)],
                "socket_power_W": pws[len(pws) // 2] if pws else None,
                "samples": len(clks), "reads": self.reads,
                "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), median of the "
                          "fresh readings under load (repeats of a reading dropped)"}


# ---------------------------------------------------------------------------
# CPU baseline
# ---------------------------------------------------------------------------

def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            return (max(p.get("num_threads", 1) for p in info),
                    ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}"
                                      for p in info})))
    except Exception:  # noqa: BLE001
        pass
    return os.cpu_count() or 1, "unknown"


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _cpu_baseline(layer, g, seed, target_s):
    """The oracle as it stands, per stage, on row chunks of the workload's up
    projection until ~target_s seconds pass: activation rotate + quantize
    (GB/s on 3 B per element + 4 B per token), dequant + derotate (GB/s on
    3 B per element), the int32 GEMM (GOPS on 2 rows N K) and the whole
    int8 forward (value, TOPS). Each stage gets about a quarter of the time."""
    import numpy as np

    import oracle
    threads, blas = _blas_info()
    m, n, k = layer.m, layer.n, layer.k
    x_rows = min(m, 2048)
    xb = layer.x()[:x_rows]
    wb = layer.w()
    wq, s_w = oracle.quantize_weights(wb, g, seed)
    budget = target_s / 4.0

    def timed(fn):
        done, el, t0 = 0.0, 0.0, time.perf_counter()
        while el < budget or done == 0:
            done += fn(int(done))
            el = time.perf_counter() - t0
            if el > 2 * budget:
                break
        return done, el

    chunk = 256

    def actq(i):
        r0 = (i % max(1, x_rows - chunk + 1))
        oracle.quantize_activations(np.ascontiguousarray(xb[r0:r0 + chunk]), g, seed)
        return min(chunk, x_rows - r0)

    def deq(i):
        r0 = (i * 7) % max(1, n - 1024 + 1)
        oracle.dequant_derotate(wq[r0:r0 + 1024], s_w, g, seed)
        return min(1024, n - r0)

    xq_s, sx_s = oracle.quantize_activations(np.ascontiguousarray(xb[:chunk]), g, seed)

    def gemm(i):
        oracle.gemm_int32(xq_s, wq)
        return xq_s.shape[0]

    def lin(i):
        r0 = (i % max(1, x_rows - chunk + 1))
        oracle.linear_int8(np.ascontiguousarray(xb[r0:r0 + chunk]), wq, s_w, g, seed)
        return min(chunk, x_rows - r0)

    a_rows, a_s = timed(actq)
    d_rows, d_s = timed(deq)
    g_rows, g_s = timed(gemm)
    l_rows, l_s = timed(lin)
    return {
        "value": round(2.0 * l_rows * n * k / l_s / 1e12, 6), "unit": "TOPS",
        "cores": int(threads), "kind": "oracle",
        "sample": f"oracle stages on row chunks of the {m}x{n}x{k} up projection "
                  f"(g={g}): act-quant {int(a_rows)} token rows in {a_s:.1f} s, dequant "
                  f"{int(d_rows)} weight rows in {d_s:.1f} s, int32 GEMM {int(g_rows)} rows in "
                  f"{g_s:.1f} s, whole forward {int(l_rows)} rows in {l_s:.1f} s",
        "stages": {
            "act_quant_GB/s": round((3.0 * k + 4.0) * a_rows / a_s / 1e9, 4),
            "dequant_GB/s": round(3.0 * k * d_rows / d_s / 1e9, 4),
            "gemm_int32_GOPS": round(2.0 * g_rows * n * k / g_s / 1e9, 2),
            "linear_TOPS": round(2.0 * l_rows * n * k / l_s / 1e12, 6)},
        "cpu_model": _cpu_model(), "blas": blas,
        "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
        else os.cpu_count(),
    }


# ---------------------------------------------------------------------------
# All workload configs (one JSON line each)
# ---------------------------------------------------------------------------

def _copies(t, footprint):
    n = 1 if footprint >= 2 * MALL_BYTES else max(2, math.ceil(2 * MALL_BYTES / footprint) + 1)
    return [t] + [t.clone() for _ in range(n - 1)]


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

    for layer, g in cases:
        print(f"[bench] config {layer.name} g={g}", file=sys.stderr, flush=True)
        r = _layer_legs(cr, layer, g, seed, to_dev(layer.x()), reps, stream, dev, with_deq=True)
        r = {"config": layer.name, "m": layer.m, "n": layer.n, "k": layer.k, "g": g, **r}
        print(json.dumps(r), flush=True)


def _layer_legs(cr, layer, g, seed, x0, reps, stream, dev, with_deq=True, w=None):
    """GEMM, linear, act-quant and dequant of one layer (HIP-event means)."""
    import torch
    m, n, k = layer.m, layer.n, layer.k
    if w is None:
        import numpy as np
        w = torch.from_numpy(layer.w().view(np.int16)).view(torch.bfloat16).to(dev)
    wq, s_w = cr.convrot_quantize_weights(w, g, seed)
    del w
    xs = _copies(x0, 3 * m * k)
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    sx = torch.empty(m, dtype=torch.float32, device=dev)
    cr.convrot_quantize_activations(x0, g, seed, xq=xq, s_x=sx)
    ys = _copies(torch.empty((m, n), dtype=torch.bfloat16, device=dev), 2 * m * n)
    ws = torch.empty(cr.convrot_linear_int8_workspace_size(m, n, k), dtype=torch.uint8,
                     device=dev)
    act_ms = _events_time(lambda i: cr.convrot_quantize_activations(
        xs[i % len(xs)], g, seed, xq=xq, s_x=sx), reps, stream)
    gemm_ms = _events_time(lambda i: cr.convrot_gemm_int8(
        xq, sx, wq, s_w, y=ys[i % len(ys)]), reps, stream)
    lin_ms = _events_time(lambda i: cr.convrot_linear_int8(
        xs[i % len(xs)], wq, s_w, g, seed, workspace=ws, out=ys[i % len(ys)]), reps, stream)
    del xs, ys, ws, xq
    ops = 2.0 * m * n * k
    act_b, deq_b = 3.0 * m * k + 4.0 * m, 3.0 * n * k + 4.0
    out = {
        "gemm_TOPS": round(ops / (gemm_ms * 1e-3) / 1e12, 1),
        "gemm_frac_peak": round(ops / (gemm_ms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        "linear_TOPS": round(ops / (lin_ms * 1e-3) / 1e12, 1),
        "act_quant_GB/s": round(act_b / (act_ms * 1e-3) / 1e9, 1),
        "act_quant_frac_hbm": round(act_b / (act_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "us": {"gemm": round(gemm_ms * 1e3, 2), "linear": round(lin_ms * 1e3, 2),
               "act_quant": round(act_ms * 1e3, 2)}}
    if with_deq:
        wqs = _copies(wq, 3 * n * k)
        outs = _copies(torch.empty((n, k), dtype=torch.bfloat16, device=dev), 3 * n * k)
        deq_ms = _events_time(lambda i: cr.convrot_dequant_derotate(
            wqs[i % len(wqs)], s_w, g, seed, out=outs[i % len(outs)]), reps, stream)
        del wqs, outs
        out["dequant_GB/s"] = round(deq_b / (deq_ms * 1e-3) / 1e9, 1)
        out["dequant_frac_hbm"] = round(deq_b / (deq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        out["us"]["dequant"] = round(deq_ms * 1e3, 2)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------
# Headline
# ---------------------------------------------------------------------------

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
    if args.leg:
        _one_leg(args)
        return

    import numpy as np
    import torch

    import int8_gemm_amd as cr
    import synth

    cr.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    seed, g = synth.ROT_SEED, 256
    up, down = synth.WAN_FFN_UP, synth.WAN_FFN_DOWN
    m = up.m
    print(f"[bench] workload wan-ffn {m} tokens, {up.k} <-> {up.n}, g={g}: generating inputs",
          file=sys.stderr, flush=True)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x1, x2 = to_dev(up.x()), to_dev(down.x())
    wq1, sw1 = cr.convrot_quantize_weights(to_dev(up.w()), g, seed)
    wq2, sw2 = cr.convrot_quantize_weights(to_dev(down.w()), g, seed)
    y1 = torch.empty((m, up.n), dtype=torch.bfloat16, device=dev)
    y2 = torch.empty((m, down.n), dtype=torch.bfloat16, device=dev)
    ws1 = torch.empty(cr.convrot_linear_int8_workspace_size(m, up.n, up.k), dtype=torch.uint8,
                      device=dev)
    ws2 = torch.empty(cr.convrot_linear_int8_workspace_size(m, down.n, down.k),
                      dtype=torch.uint8, device=dev)

    def step(i):
        cr.convrot_linear_int8(x1, wq1, sw1, g, seed, workspace=ws1, out=y1)
        cr.convrot_linear_int8(x2, wq2, sw2, g, seed, workspace=ws2, out=y2)

    # warm-up: the given steps, and at least STEP_WARM_MS of them (the clocks
    # settle over the first ~10 ms of load)
    print("[bench] warmup", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    i = 0
    while i < args.warmup or (time.perf_counter() - t0) * 1e3 < STEP_WARM_MS:
        step(i)
        i += 1
        if i % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_steps = i
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / max(args.steps, 1)
    ops_up, ops_down = 2.0 * m * up.n * up.k, 2.0 * m * down.n * down.k
    value = (ops_up + ops_down) / (ms_step * 1e-3) / 1e12

    # ---- the roofline kernel: the up projection's GEMM as one launch ----
    print("[bench] roofline GEMM", file=sys.stderr, flush=True)
    reps = 20
    xq1 = torch.empty((m, up.k), dtype=torch.int8, device=dev)
    sx1 = torch.empty(m, dtype=torch.float32, device=dev)
    cr.convrot_quantize_activations(x1, g, seed, xq=xq1, s_x=sx1)
    gemm_ms = _events_time(lambda i: cr.convrot_gemm_int8(xq1, sx1, wq1, sw1, y=y1), reps, stream)
    sampler = ClockSampler()

    def clock_run():  # ~2 s of the same GEMM while the sampler reads the clock
        for i in range(max(1, int(2000.0 / max(gemm_ms, 1e-3)))):
            cr.convrot_gemm_int8(xq1, sx1, wq1, sw1, y=y1)
            if i % 50 == 49:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    sampler.run_during(clock_run)
    clock = sampler.summary()
    gemm_tops = ops_up / (gemm_ms * 1e-3) / 1e12
    plan = cr.convrot_plan_launch("gemm", m=m, n=up.n, k=up.k)
    roofline = {
        "bound": "mfma", "kernel": "gemm_i8_kernel",
        "tile": f"{plan['tile_m']}x{plan['tile_n']}", "grid_workgroups": plan["grid"],
        "shape": f"{m}x{up.n}x{up.k}",
        "achieved": round(gemm_tops, 3), "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
        "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
        "traffic": _traffic(1),
        "algorithmic_bytes": float(m * up.k + up.n * up.k + 2 * m * up.n + 4 * m),
        "avg_ms": round(gemm_ms, 5), "batches": 3, "launches_per_batch": reps,
        **clock}
    if clock.get("sclk_MHz"):
        peak_clk = NUM_CUS * INT8_OPS_PER_CLK_PER_CU * clock["sclk_MHz"] * 1e6 / 1e12
        roofline["peak_at_sclk"] = round(peak_clk, 1)
        roofline["frac_at_sclk"] = round(gemm_tops / peak_clk, 4)
    torch.cuda.synchronize()

    # ---- each leg: linear, GEMM, act-quant, dequant ----
    print("[bench] legs", file=sys.stderr, flush=True)
    legs = {}
    for name, lay, x in (("up", up, x1), ("down", down, x2)):
        legs[name] = {"shape": f"{lay.m}x{lay.n}x{lay.k}",
                      **_layer_legs(cr, lay, g, seed, x, 10, stream, dev, with_deq=True)}
    del xq1, sx1, ws1, ws2
    torch.cuda.synchronize()

    result = {
        "metric": "int8 convrot linear TOPS (+% int8 MFMA peak); dequant/act-quant GB/s "
                  "(+% HBM)",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"wan-ffn pair: x1 bf16 [{m},{up.k}] -> W1 int8 "
                               f"[{up.n},{up.k}] and x2 bf16 [{m},{down.k}] -> W2 int8 "
                               f"[{down.n},{down.k}], N(0,1) activations, Gaussian weights "
                               "with 1% Student-t(3) outlier columns, g=256, R = "
                               "Walsh-Hadamard x seeded signs, default workspace",
                   "m": m, "n_up": up.n, "k_up": up.k, "g": g, "rot_seed": seed},
        "roofline": roofline,
        "legs": legs,
        "linear_tops_frac_peak": round(value / PEAK_INT8_TOPS, 4),
    }
    if not args.headline_only:
        del x1, x2, y1, y2
        torch.cuda.empty_cache()
        result.update(_extras(cr, dev, stream, seed, to_dev))
    if args.calibrate_copy:  # three plain 1 GiB copies for the counter calibration
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = _cpu_baseline(up, g, seed, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _extras(cr, dev, stream, seed, to_dev):
    """Other shapes and paths: the Z-Image attention projection, its
    per-channel and FP16 forms, the 60-layer dequant stack, the same stack
    streamed from host memory, and the device copy ceiling."""
    import numpy as np
    import torch

    import synth
    g = 256
    out = {}
    reps = 50
    # ---- Z-Image attention projection (4608 tokens) ----
    print("[bench] zimage-attn", file=sys.stderr, flush=True)
    layer = synth.ZIMAGE_ATTN
    m, n, k = layer.m, layer.n, layer.k
    x0 = to_dev(layer.x())
    w = to_dev(layer.w())
    out["zimage_attn"] = {"shape": f"{m}x{n}x{k}",
                          **_layer_legs(cr, layer, g, seed, x0, reps, stream, dev, w=w.clone())}
    xs = _copies(x0, 3 * m * k)
    ws = torch.empty(cr.convrot_linear_int8_workspace_size(m, n, k), dtype=torch.uint8,
                     device=dev)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    ops = 2.0 * m * n * k
    wq, s_w = cr.convrot_quantize_weights(w, g, seed)
    xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    sx = torch.empty(m, dtype=torch.float32, device=dev)
    cr.convrot_quantize_activations(x0, g, seed, xq=xq, s_x=sx)
    tiles = {}
    for t in (128, 192, 256, 384):
        t_ms = _events_time(lambda i: cr.convrot_gemm_int8(xq, sx, wq, s_w, y=y, tile=t), reps,
                            stream)
        tiles[str(t)] = round(ops / (t_ms * 1e-3) / 1e12, 1)
    out["zimage_attn"]["gemm_TOPS_by_forced_tile"] = tiles

    # ---- per-output-channel weight scales ----
    wq_pc, sw_pc = cr.convrot_quantize_weights_per_channel(w, g, seed)
    nrot_w = max(2, math.ceil(2 * MALL_BYTES / (3 * n * k)) + 1)
    outs = [torch.empty((n, k), dtype=torch.bfloat16, device=dev) for _ in range(nrot_w)]
    pc_lin = _events_time(lambda i: cr.convrot_linear_int8_per_channel(
        xs[i % len(xs)], wq_pc, sw_pc, g, seed, workspace=ws, out=y), reps, stream)
    pc_gemm = _events_time(lambda i: cr.convrot_gemm_int8_per_channel(
        xq, sx, wq_pc, sw_pc, y=y), reps, stream)
    wqs_pc = [wq_pc] + [wq_pc.clone() for _ in range(nrot_w - 1)]
    pc_deq = _events_time(lambda i: cr.convrot_dequant_derotate_per_channel(
        wqs_pc[i % nrot_w], sw_pc, g, seed, out=outs[i % nrot_w]), reps, stream)
    out["per_channel"] = {
        "shape": f"{m}x{n}x{k}",
        "linear_TOPS": round(ops / (pc_lin * 1e-3) / 1e12, 1),
        "gemm_TOPS": round(ops / (pc_gemm * 1e-3) / 1e12, 1),
        "gemm_frac_peak": round(ops / (pc_gemm * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        "dequant_GB/s": round((3.0 * n * k + 4.0 * n) / (pc_deq * 1e-3) / 1e9, 1),
        "dequant_frac_hbm": round((3.0 * n * k + 4.0 * n) / (pc_deq * 1e-3) / 1e9
                                  / PEAK_HBM_GBS, 4)}
    del wqs_pc, outs, wq_pc

    # ---- FP16 activations and outputs ----
    xh0 = torch.from_numpy(layer.x(fmt="f16").view(np.int16)).view(torch.float16).to(dev)
    xhs = _copies(xh0, 3 * m * k)
    yh = torch.empty((m, n), dtype=torch.float16, device=dev)
    h_lin = _events_time(lambda i: cr.convrot_linear_int8_ex(
        xhs[i % len(xhs)], wq, s_w, g, seed, workspace=ws, out=yh), reps, stream)
    h_act = _events_time(lambda i: cr.convrot_quantize_activations_ex(
        xhs[i % len(xhs)], g, seed, xq=xq, s_x=sx), reps, stream)
    act_bytes = 3.0 * m * k + 4.0 * m
    out["f16"] = {"shape": f"{m}x{n}x{k}",
                  "linear_TOPS": round(ops / (h_lin * 1e-3) / 1e12, 1),
                  "act_quant_GB/s": round(act_bytes / (h_act * 1e-3) / 1e9, 1),
                  "act_quant_frac_hbm": round(act_bytes / (h_act * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                              4)}
    del xhs, xh0, yh, xs, x0, w
    torch.cuda.synchronize()

    # ---- dequant over the 60-layer stack: 60 + 60 distinct int8 buffers of
    # the two stack shapes and as many outputs, one dequant each per pass ----
    print("[bench] dequant stack", file=sys.stderr, flush=True)
    stack = []
    for lay in (synth.STACK_SQUARE, synth.STACK_WIDE):
        wq_l, sw_l = cr.convrot_quantize_weights(to_dev(lay.w()), g, seed)
        copies = [wq_l.clone() for _ in range(synth.STACK_LAYERS)]
        del wq_l
        outs_l = [torch.empty((lay.n, lay.k), dtype=torch.bfloat16, device=dev)
                  for _ in range(synth.STACK_LAYERS)]
        stack.append((copies, sw_l, outs_l))

    order = [(layer_i, si) for layer_i in range(synth.STACK_LAYERS) for si in range(2)]
    b_wqs = [stack[si][0][layer_i] for layer_i, si in order]
    b_sws = [stack[si][1] for layer_i, si in order]
    b_outs = [stack[si][2][layer_i] for layer_i, si in order]

    def stack_pass(i):  # one batched call: the 120 weights in launches of 48
        cr.convrot_dequant_derotate_batched(b_wqs, b_sws, g, seed, outs=b_outs)

    def stack_pass_per_layer(i):  # one call per weight
        for layer_i, si in order:
            cr.convrot_dequant_derotate(stack[si][0][layer_i], stack[si][1], g, seed,
                                        out=stack[si][2][layer_i])

    stack_ms = _events_time(stack_pass, 3, stream)
    per_layer_ms = _events_time(stack_pass_per_layer, 3, stream)
    stack_bytes = float(sum(3 * c[0].numel() * len(c) + 4 * len(c) for c, _, _ in stack))
    out["dequant_stack"] = {
        "layers": 2 * synth.STACK_LAYERS, "call": "convrot_dequant_derotate_batched",
        "GB/s": round(stack_bytes / (stack_ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(stack_bytes / (stack_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "ms_per_pass": round(stack_ms, 4), "bytes": stack_bytes,
        "per_layer_calls_ms_per_pass": round(per_layer_ms, 4),
        "per_layer_calls_frac_hbm": round(stack_bytes / (per_layer_ms * 1e-3) / 1e9
                                          / PEAK_HBM_GBS, 4)}
    del b_outs
    for _, _, outs_l in stack:
        outs_l.clear()
    torch.cuda.empty_cache()

    # ---- the same stack streamed from pinned host memory: 4608 tokens
    # through every layer, each layer's int8 weight copied to the GPU on the
    # streamer's copy stream while earlier layers compute ----
    print("[bench] streamed stack", file=sys.stderr, flush=True)
    sm_tok = layer.m
    xs_k = to_dev(synth.activations(sm_tok, synth.STACK_SQUARE.k, 505))
    host_layers, dev_layers = [], []
    for layer_i in range(synth.STACK_LAYERS):
        for copies, sw_l, _ in stack:
            host_layers.append((copies[layer_i].cpu().pin_memory(), sw_l))
            dev_layers.append((copies[layer_i], sw_l))
    stream_bytes = float(sum(w_.numel() for w_, _ in host_layers))
    ys = {n_: torch.empty((sm_tok, n_), dtype=torch.bfloat16, device=dev)
          for n_ in {w_.shape[0] for w_, _ in host_layers}}
    ws_s = torch.empty(max(cr.convrot_linear_int8_workspace_size(sm_tok, n_, xs_k.shape[1])
                           for n_ in ys), dtype=torch.uint8, device=dev)
    slot_bytes = max(w_.numel() for w_, _ in host_layers)
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
    str_ms = _events_time(streamed_pass, 2, stream)
    res_ms = _events_time(resident_pass, 2, stream)
    cpy_ms = _events_time(copy_pass, 2, stream)
    streamer.close()
    stack_ops = float(sum(2.0 * sm_tok * w_.shape[0] * w_.shape[1] for w_, _ in host_layers))
    out["streamed_stack"] = {
        "layers": 2 * synth.STACK_LAYERS, "tokens": sm_tok,
        "int8_bytes_per_pass": stream_bytes,
        "ms_per_pass": round(str_ms, 3),
        "h2d_GB/s": round(stream_bytes / (str_ms * 1e-3) / 1e9, 1),
        "copy_only_ms": round(cpy_ms, 3),
        "copy_only_GB/s": round(stream_bytes / (cpy_ms * 1e-3) / 1e9, 1),
        "frac_of_copy_only": round(cpy_ms / str_ms, 4),
        "resident_ms_per_pass": round(res_ms, 3),
        "resident_TOPS": round(stack_ops / (res_ms * 1e-3) / 1e12, 1),
        "streamed_TOPS": round(stack_ops / (str_ms * 1e-3) / 1e12, 1)}
    del stack, host_layers, dev_layers, ys, ws_s, staging, xs_k
    torch.cuda.synchronize()

    # ---- the device's copy ceiling: a plain 1 GiB copy, read + write bytes ----
    print("[bench] copy ceiling", file=sys.stderr, flush=True)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cp_ms = _events_time(lambda i: dst.copy_(src), 5, stream)
    out["copy_ceiling"] = {"bytes_per_copy": 2.0 * (1 << 30),
                           "GB/s": round(2.0 * (1 << 30) / (cp_ms * 1e-3) / 1e9, 1),
                           "frac_hbm": round(2.0 * (1 << 30) / (cp_ms * 1e-3) / 1e9
                                             / PEAK_HBM_GBS, 4),
                           "kernel": "torch copy_ (device to device), HIP-event mean"}
    del src, dst
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    main()
