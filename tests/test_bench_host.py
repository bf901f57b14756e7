"""bench.py's contract on the CPU: the one-GPU refusal happens before anything
touches a GPU, the options exist, the CPU-baseline leg reports the fields the
JSON line carries, and the HBM traffic figure is only taken from a counter
summary made on the current GEMM source."""

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
