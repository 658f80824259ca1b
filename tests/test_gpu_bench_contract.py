"""bench.py's one-line JSON output on the GPU: the keys the benchmark contract names,
with consistent values, on a short run of the smallest workloads."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print(f"[bench contract] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def test_bench_json_contract():
    d = run_bench("--workload", "qwen3_8b_packed", "--steps", "5", "--warmup", "2",
                  "--cpu-seconds", "0.5")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "per_config"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "qwen3_8b_packed" and d["value"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert abs(r["achieved"] - r["bytes_per_launch"] / (r["avg_launch_us"] * 1e-6) / 1e9) < 1e-6
    assert 0.3 < r["frac"] < 1.0 and r["frac_of_ceiling"] > 0
    assert r["launches_per_pass"] == 1
    assert abs(r["avg_pass_us"] - r["avg_launch_us"] * r["launches_per_pass"]) < 1e-6
    step_gbps = 2 * r["bytes_per_launch"] * r["launches_per_pass"] / (d["ms_per_step"] * 1e-3) / 1e9
    assert abs(d["step_hbm_GBps"] - step_gbps) < 1e-6 * step_gbps
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    assert set(d["per_config"]) == {"tiny_packed", "qwen3_4b_packed", "qwen3_8b_packed",
                                    "qwen3_8b_padded", "qwen3_32b_packed", "long_ctx_512k"}
    assert d["per_config"]["qwen3_8b_packed"].get("headline") is True
    long = d["per_config"]["long_ctx_512k"]  # 2621440 workgroups: 8 launches per pass
    assert long["launches_per_pass"] == 8 and long["index"] == "64-bit"
    assert abs(long["avg_pass_us"] - 8 * long["avg_launch_us"]) < 1e-6
    pad = d["per_config"]["qwen3_8b_padded"]
    assert pad["padded_launch"] == "compact" and pad["kernel"] == "rope_qk_group_kernel"
    assert 0.8 < pad["t_over_packed"] < 1.5 and pad["valid_fraction"] < 0.6
    assert pad["seqused_kernel"] == "rope_qk_kernel" and pad["seqused_launch_us"] > 0


def test_bench_json_multi_launch_pass():
    """The 524288-token workload, whose passes are 8 launches: per-launch and per-pass
    figures consistent with each other and with the step time, the traffic (when the
    committed counter summary matches the sources) per launch."""
    d = run_bench("--workload", "long_ctx_512k", "--configs", "none", "--steps", "3",
                  "--warmup", "1", "--cpu-seconds", "0.5")
    r = d["roofline"]
    assert d["config"]["workload"] == "long_ctx_512k" and r["launches_per_pass"] == 8
    assert r["bytes_per_launch"] == 524288 * 20480 // 8
    assert abs(r["avg_pass_us"] - 8 * r["avg_launch_us"]) < 1e-6 * r["avg_pass_us"]
    assert abs(r["achieved"] - r["bytes_per_launch"] / (r["avg_launch_us"] * 1e-6) / 1e9) < 1e-6
    step_gbps = 2 * r["bytes_per_launch"] * 8 / (d["ms_per_step"] * 1e-3) / 1e9
    assert abs(d["step_hbm_GBps"] - step_gbps) < 1e-6 * step_gbps
    assert 0.5 < r["frac"] < 1.0
    assert r["traffic"] is None or abs(r["traffic"] / r["bytes_per_launch"] - 1) < 0.01
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0
