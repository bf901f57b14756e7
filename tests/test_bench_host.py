"""bench.py's contract on the CPU: the one-GPU refusal happens before anything
touches a GPU, the options exist, the CPU-baseline leg reports the fields the
JSON line carries, the HBM traffic figure is only taken from a counter
summary made on the current GEMM source, and the clock sampler keeps fresh
readings only."""

import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    for argv in (["--gpus", "2"], ["--gpus", "8", "--all-configs"]):
        r = _run(*argv)
        assert r.returncode == 2
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--all-configs", "--warm-ms", "--no-cpu-baseline",
                "--calibrate-copy", "--headline-only"):
        assert opt in r.stdout, opt


def test_cpu_baseline_fields():
    res = bench._cpu_baseline(synth.TINY, 256, synth.ROT_SEED, 0.4)
    assert {"value", "unit", "cores", "kind", "sample", "stages", "cpu_model", "blas"} <= set(res)
    assert res["kind"] == "oracle" and res["unit"] == "TOPS"
    assert res["value"] > 0 and res["cores"] >= 1
    assert "64x256x256" in res["sample"]
    st = res["stages"]
    for key in ("act_quant_GB/s", "dequant_GB/s", "gemm_int32_GOPS", "linear_TOPS"):
        assert st[key] > 0, key
    assert st["linear_TOPS"] == res["value"]
    assert res["cpu_model"] and res["blas"]


def test_traffic_only_for_the_current_gemm_source(tmp_path, monkeypatch):
    cur = bench._source_hash(bench.GEMM_SOURCE)
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({"gemm_source_sha256_16": cur, "hbm_bytes_per_launch": 1234}))
    assert bench._traffic(1) == 1234
    f.write_text(json.dumps({"gemm_source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 1234}))
    assert bench._traffic(1) is None
    f.write_text("not json")
    assert bench._traffic(1) is None


def test_clock_sampler_keeps_fresh_readings_only():
    """A firmware figure that repeats is stale: only readings that differ
    from the one before them (after the settle time) enter the median."""
    class FakeSmi:
        def __init__(self, seq):
            self.seq, self.i = seq, 0

        def amdsmi_get_gpu_metrics_info(self, handle):
            clk, pw = self.seq[min(self.i, len(self.seq) - 1)]
            self.i += 1
            return {"current_gfxclks": [clk] * 8, "current_socket_power": pw}

    s = bench.ClockSampler.__new__(bench.ClockSampler)
    s.settle_s, s.period_s = 0.0, 0.0
    s.samples, s.error, s._last, s.reads = [], None, None, 0
    seq = [(2100, 800)] * 5 + [(1700, 1350)] + [(1700, 1350)] * 3 + [(1750, 1340)] + [(1650, 1380)] * 4
    s._amdsmi, s._handle = FakeSmi(seq), object()
    s._stop = bench.threading.Event()
    calls = {"n": 0}
    real_wait = s._stop.wait

    def stop_after(timeout):  # end the loop once the sequence is read
        calls["n"] += 1
        if calls["n"] >= len(seq):
            s._stop.set()
        return real_wait(0)

    s._stop.wait = stop_after
    s._run()
    got = s.summary()
    assert s.reads == len(seq)
    assert [c for c, _ in s.samples] == [2100, 1700, 1750, 1650]
    assert got["sclk_MHz"] == 1750 and got["samples"] == 4
