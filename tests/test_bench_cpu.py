"""bench.py without a GPU: the one-GPU guard, the work it credits per block,
and the bookkeeping that keeps stale HBM counters out of its roofline."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from video_audio_diffusion_ltxattn_amd import synth  # noqa: E402


def run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_headline_work_matches_closed_forms():
    """4*B*H*Sq*Sk*D per kind at 15360 video / 126 valid audio keys, H32 D128:
    3865.5 GFLOP video self (98% of the block), 31.7 GFLOP for each cross kind."""
    w = synth.WORKLOADS[3]
    f = synth.attention_flops(w)
    assert f["video_self"] == 4 * 32 * 15360 * 15360 * 128
    assert f["a2v"] == f["v2a"] * 126 / 128 == 4 * 32 * 15360 * 126 * 128
    assert f["audio_self"] == 4 * 32 * 128 * 126 * 128
    assert abs(f["video_self"] / 1e9 - 3865.5) < 0.1
    assert 0.98 < f["video_self"] / sum(f.values()) < 0.99
    b = synth.attention_bytes(w)
    assert b["video_self"] == 4 * 15360 * 32 * 128 * 2                 # Q, K, V, O once
    assert b["a2v"] == b["v2a"] == (2 * 15360 + 2 * 128) * 32 * 128 * 2


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() {\n  return 1;  // one\n}\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.kernel_source_hash()
    src.write_text("int f() {\n\n  return 1;  // another comment\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_only_for_the_code_it_was_taken_on(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    traffic = tmp_path / "t.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    w = synth.WORKLOADS[3]
    assert bench.measured_traffic(w) is None                      # no file
    traffic.write_text(json.dumps({"kernel_source_sha256_16": bench.kernel_source_hash(),
                                   "workload": bench.workload_key(w), "bytes_per_launch": 123}))
    assert bench.measured_traffic(w) == 123
    assert bench.measured_traffic(synth.WORKLOADS[2]) is None     # taken on another workload
    src.write_text("int f() { return 2; }\n")                    # the kernel changed since
    assert bench.measured_traffic(w) is None
    traffic.write_text("{not json")
    assert bench.measured_traffic(w) is None


def test_committed_traffic_file_names_its_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert len(t["kernel_source_sha256_16"]) == 16
    assert t["bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    assert t["workload"] == bench.workload_key(synth.WORKLOADS[3])   # the headline workload


def test_roofline_kernel_name_follows_the_shape():
    assert bench.video_kernel_name(synth.WORKLOADS[3]).startswith("fa_ring_kernel<128, 8, 1>")
    assert not bench.video_kernel_name(synth.WORKLOADS[1]).startswith("fa_ring_kernel")   # 256 tokens, D = 64
