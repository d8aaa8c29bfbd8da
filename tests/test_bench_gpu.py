"""bench.py end to end on the GPU, on the tiny block: one JSON line with the
fields the benchmark contract names, roofline and CPU baseline included."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--cfg", "1", "--steps", "3",
                        "--warmup", "2", "--kind-calls", "2", *args],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_json_line():
    d = run_bench("--cpu-seconds", "0.5")
    assert d["value"] > 0 and d["unit"] == "TFLOP/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["ms_per_step"] > 0 and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("LTX-2 block attention set")
    assert set(d["kinds"]) == {"video_self", "audio_self", "a2v", "v2a"}
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 2500.0
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-4
    assert rl["traffic"] is None   # the committed counters are for the headline workload only
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["one_core_value"] > 0


@pytest.mark.gpu
@pytest.mark.parametrize("flag", ["--overlap", "--distinct", "--gated", "--qknorm-rope"])
def test_bench_modes(flag):
    d = run_bench("--no-cpu-baseline", flag)
    assert d["value"] > 0 and "cpu_baseline" not in d
    if flag == "--qknorm-rope":
        p = d["qknorm_rope"]
        assert d["config"]["qk_prologue"] is True
        assert p["fused_block_ms"] > 0 and p["unfused_torch_block_ms"] > 0 and p["plain_block_ms"] > 0
