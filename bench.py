#!/usr/bin/env python3
"""Benchmark: attention TFLOP/s of one LTX-2 DiT block's attention set on one MI355X.

A step is one ``ltxattn_block_attention`` call -- video self-attention, v2a
(key-range pass + combine), a2v and audio self-attention -- over the
768x1280x121 clip: 15360 video tokens, 126 audio tokens padded to 128, 32
heads of 128, batch 1 (TensorRT-LLM PR #16228, "Description").  Inputs are
seeded synthetic bf16 tensors already resident in HBM.

Prints one JSON line.  ``value`` is the block's algorithmic attention FLOPs
(4*B*H*Sq*Sk_valid*D summed over the four kinds) per second of step time.
``roofline`` describes the dominant kernel (video self-attention), timed
with HIP events the library records on the stream it launches on; in the
timed region only that kind's events are recorded.  ``kinds`` comes from a
separate, untimed pass that records every kind's boundaries.
``cpu_baseline`` is the double-precision oracle on a bounded sample of the
same work on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from video_audio_diffusion_ltxattn_amd import synth  # noqa: E402

METRIC = "attention TFLOP/s + % bf16 MFMA peak per DiT block (15360 video/126 audio tok)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KINDS = ("video_self", "audio_self", "a2v", "v2a")
KERNEL_SRC = os.path.join(ROOT, "video_audio_diffusion_ltxattn_amd", "csrc", "ltxattn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_video_self_15360.json")


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel source's code: comments, blank lines and
    trailing blanks are dropped, so only a change of code invalidates the
    counters taken on it."""
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def workload_key(w: synth.Workload) -> str:
    return f"video {w.video_len}, H{w.heads}, D{w.head_dim}, B{w.batch}"


def measured_traffic(w: synth.Workload):
    """HBM bytes per video-self launch from the committed rocprofv3 counter
    runs, or None if they were taken on a different kernel source or a
    different workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload_key(w):
        return None
    return t.get("bytes_per_launch")


def video_kernel_name(w: synth.Workload) -> str:
    """The kernel video self-attention runs on for this shape (the library's
    choice: the ring kernel for long sequences at D = 128)."""
    if w.head_dim == 128 and w.video_len >= 1024:
        return "fa_ring_kernel<128, 8, 1> (video self-attention)"
    return "video self-attention kernel (fa_kvres_kernel or fa_fwd_kernel at this shape)"


def cpu_baseline(inputs: dict, w: synth.Workload, min_s: float, max_s: float) -> dict:
    """The oracle, as it stands, on video self-attention rows of the same inputs:
    whole rows (all keys), in chunks, until at least min_s seconds have passed."""
    import oracle
    threads = oracle.default_threads()
    q, k, v = inputs["video_q"], inputs["video_k"], inputs["video_v"]
    rng = np.random.default_rng(0)
    chunk = 8 * threads
    rows_done = 0
    t0 = time.perf_counter()
    elapsed = 0.0
    while elapsed < min_s:
        rows = np.stack([rng.integers(0, w.batch, chunk), rng.integers(0, w.heads, chunk),
                         rng.integers(0, w.video_len, chunk)], axis=1)
        oracle.attention_rows(q, k, v, rows, threads=threads)
        rows_done += chunk
        elapsed = time.perf_counter() - t0
        if elapsed > max_s:
            break
    flops = 4.0 * rows_done * w.video_len * w.head_dim
    # The same on one thread, briefly: the per-core figure.
    rows1, t1, el1 = 0, time.perf_counter(), 0.0
    while el1 < min_s / 4:
        rows = np.stack([rng.integers(0, w.batch, 8), rng.integers(0, w.heads, 8),
                         rng.integers(0, w.video_len, 8)], axis=1)
        oracle.attention_rows(q, k, v, rows, threads=1)
        rows1 += 8
        el1 = time.perf_counter() - t1
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{rows_done} random video self-attention query rows of the block workload "
                   f"(each over all {w.video_len} keys, D={w.head_dim}), double precision, "
                   f"{elapsed:.1f} s"),
        "one_core_value": 4.0 * rows1 * w.video_len * w.head_dim / el1 / 1e12,
    }


def torch_prologue(x, w, cos, sin, eps, pairing):
    """The QK-norm + rotary prologue as separate torch operations in fp32 (the
    unfused passes a caller would otherwise run before the block call), for
    comparison only."""
    import torch
    P = x.shape[-1] // 2
    xf = x.float()
    y = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + eps) * w
    ya, yc = (y[..., :P], y[..., P:]) if pairing == "half" else (y[..., 0::2], y[..., 1::2])
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    za, zc = ya * c - yc * s, ya * s + yc * c
    z = torch.cat([za, zc], -1) if pairing == "half" else torch.stack([za, zc], -1).flatten(-2)
    return z.to(torch.bfloat16)


def prologue_comparison(lt, ba, dev, outs, w, dpros, stream, calls):
    """Block time with the prologue fused (query loads + one pass per distinct
    keys), against the same attention after separate torch passes over every
    kind's queries and keys, and against the block with no prologue."""
    import torch
    q_of = {"video_self": "video_q", "audio_self": "audio_q", "a2v": "video_q", "v2a": "audio_q"}
    k_of = {"video_self": "video_k", "audio_self": "audio_k", "a2v": "audio_k", "v2a": "video_k"}
    v_of = {"video_self": "video_v", "audio_self": "audio_v", "a2v": "audio_v", "v2a": "video_v"}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(calls):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls

    io_fused = ba.make_io(dev, w.audio_kv_len, outs, prologues=dpros)
    io_plain = ba.make_io(dev, w.audio_kv_len, outs)
    fused = timed(lambda: lt.ltxattn_block_attention(ba.handle, io_fused, stream.cuda_stream))
    plain = timed(lambda: lt.ltxattn_block_attention(ba.handle, io_plain, stream.cuda_stream))
    keep = {}

    def unfused():
        ins = {}
        done = {}
        for k in outs:
            p = dpros[k]
            kk = (k_of[k], id(p["k_weight"]))
            if kk not in done:
                done[kk] = torch_prologue(dev[k_of[k]], p["k_weight"], p["k_cos"], p["k_sin"], p["eps"], p["pairing"])
            q = torch_prologue(dev[q_of[k]], p["q_weight"], p["q_cos"], p["q_sin"], p["eps"], p["pairing"])
            ins[k] = (q, done[kk], dev[v_of[k]])
        keep["io"] = ba.make_io(dev, w.audio_kv_len, outs, inputs=ins)
        keep["ins"] = ins
        lt.ltxattn_block_attention(ba.handle, keep["io"], stream.cuda_stream)
    unfused_ms = timed(unfused)
    return {"fused_block_ms": round(fused, 4), "unfused_torch_block_ms": round(unfused_ms, 4),
            "plain_block_ms": round(plain, 4),
            "fused_overhead_ms": round(fused - plain, 4), "unfused_overhead_ms": round(unfused_ms - plain, 4),
            "pairing": next(iter(dpros.values()))["pairing"],
            "note": "prologue on every kind: per-kind q weights, k weights shared by the kinds that read "
                    "the same keys (one key pass per stream); unfused = torch fp32 ops per tensor, then the "
                    "plain block on their bf16 outputs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed block calls first: a process's first ~12 calls run up to 20%% slower "
                         "while the clocks ramp up")
    ap.add_argument("--cfg", type=int, default=3, help="workload (1..5); 3 is the headline block")
    ap.add_argument("--overlap", action="store_true",
                    help="ltxattn_block_attention_overlap: the audio-side kinds on a second stream")
    ap.add_argument("--distinct", action="store_true",
                    help="give every kind its own copies of its Q/K/V (no kind reads another's inputs "
                         "through the caches)")
    ap.add_argument("--gated", action="store_true",
                    help="gated attention: every kind's output multiplied by a gate of its shape "
                         "(uniform in (0, 1), bf16)")
    ap.add_argument("--qknorm-rope", action="store_true",
                    help="QK-norm + rotary prologue on every kind (raw Q/K in, normed and rotated inside); "
                         "also times the same attention after unfused torch passes")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write this many MiB of scratch between block calls (past the last-level "
                         "cache); value then comes from the library's per-call events")
    ap.add_argument("--kind-calls", type=int, default=20,
                    help="untimed block calls, after the timed ones, that give the per-kind times")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: "
                         "the reference for scaling HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(no sharding, no collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": 3}), flush=True)
        return
    from video_audio_diffusion_ltxattn_amd import ltxattn as lt

    w = synth.WORKLOADS[args.cfg]
    inputs = synth.make_block_inputs(w)
    dev = {}
    for n, a in inputs.items():
        dev[n] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to("cuda:0")
    ba = lt.BlockAttention(w.heads, w.head_dim, w.batch, w.video_len, w.audio_len, qk_prologue=args.qknorm_rope)
    outs = {k: torch.empty_like(dev["video_q"] if k in ("video_self", "a2v") else dev["audio_q"])
            for k in KINDS}
    stream = torch.cuda.current_stream()
    kind_inputs = None
    if args.distinct:
        pairs = {"video_self": ("video_q", "video_k", "video_v"), "audio_self": ("audio_q", "audio_k", "audio_v"),
                 "a2v": ("video_q", "audio_k", "audio_v"), "v2a": ("audio_q", "video_k", "video_v")}
        kind_inputs = {k: tuple(dev[n].clone() for n in names) for k, names in pairs.items()}
    gates = None
    if args.gated:
        gates = {k: (torch.rand_like(outs[k], dtype=torch.float32) * 0.999 + 0.0005).to(torch.bfloat16)
                 for k in KINDS}
    dpros = None
    if args.qknorm_rope:
        pros = synth.make_prologues(w, "half", shared_k=True)
        seen = {}   # one device copy per distinct array: kinds sharing keys share one key pass
        for p in pros.values():
            for n, v in p.items():
                if isinstance(v, np.ndarray) and id(v) not in seen:
                    seen[id(v)] = torch.from_numpy(v).to("cuda:0")
        dpros = {k: {n: seen.get(id(v), v) for n, v in p.items()} for k, p in pros.items()}
    io = ba.make_io(dev, w.audio_kv_len, outs, kind_inputs, gates, dpros)
    scratch = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device="cuda:0")
               if args.flush_mib else None)

    block = lt.ltxattn_block_attention_overlap if args.overlap else lt.ltxattn_block_attention
    for i in range(args.warmup):
        if scratch is not None:
            scratch.fill_(float(i))
        block(ba.handle, io, stream.cuda_stream)
    torch.cuda.synchronize()

    # Timed region: events only around video self-attention (3 per call),
    # enough for the roofline's kernel time; with a flush between calls the
    # whole call is timed by its events, so every kind is recorded.
    if scratch is not None:
        lt.ltxattn_profile_begin(ba.handle, args.steps)
    else:
        lt.ltxattn_profile_begin_kinds(ba.handle, args.steps, ["video_self"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.fill_(float(i))
        block(ba.handle, io, stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    rec = lt.ltxattn_profile_read(ba.handle, args.steps)
    lt.ltxattn_profile_end(ba.handle)
    # Per-kind breakdown: a separate pass with every kind's boundaries recorded.
    if scratch is None:
        lt.ltxattn_profile_begin(ba.handle, args.kind_calls)
        for i in range(args.kind_calls):
            block(ba.handle, io, stream.cuda_stream)
        torch.cuda.synchronize()
        rec_kinds = lt.ltxattn_profile_read(ba.handle, args.kind_calls)
        lt.ltxattn_profile_end(ba.handle)
    else:
        rec_kinds = rec

    for k in KINDS:
        assert torch.isfinite(outs[k].float()).all(), f"{k}: non-finite output"

    flops = synth.attention_flops(w)
    nbytes = synth.attention_bytes(w)
    if args.gated:   # the gate is read once, like the output is written once
        qrows = {"video_self": w.video_len, "audio_self": w.audio_len, "a2v": w.video_len, "v2a": w.audio_len}
        for k in KINDS:
            nbytes[k] += 2 * w.batch * qrows[k] * w.heads * w.head_dim
    ms_step = wall * 1e3 / args.steps
    if scratch is not None:   # the flush is not the block's work: time the calls by their events
        ms_step = float(np.mean([r["total"] for r in rec]))
    value = sum(flops.values()) / (ms_step * 1e-3) / 1e12
    kind_ms = {k: float(np.mean([r[k] for r in rec_kinds])) for k in KINDS}
    kernel_ms = {k: float(np.mean([r["kernel"][k] for r in rec_kinds])) for k in KINDS}
    kinds = {}
    for k in KINDS:
        t = kind_ms[k] * 1e-3
        per_call = [r[k] for r in rec_kinds]
        kinds[k] = {"ms": round(kind_ms[k], 5),
                    "median_ms": round(float(np.median(per_call)), 5),
                    "min_ms": round(float(np.min(per_call)), 5),
                    "attention_kernels_ms": round(kernel_ms[k], 5),
                    "tflops": round(flops[k] / t / 1e12, 2),
                    "pct_bf16_peak": round(100 * flops[k] / t / 1e12 / PEAK_BF16_TFLOPS, 2),
                    "hbm_gbs": round(nbytes[k] / t / 1e9, 1),
                    "pct_hbm_peak": round(100 * nbytes[k] / t / 1e9 / PEAK_HBM_GBS, 2)}
    # The attention kernel alone (its tail combine excluded), timed region
    vs_ms = float(np.mean([r["kernel"]["video_self"] for r in rec]))
    achieved = flops["video_self"] / (vs_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, masked audio keys poisoned)",
        "config": {"workload": f"LTX-2 block attention set, {w.name}",
                   "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "video_tokens": w.video_len, "audio_tokens": w.audio_kv_len,
                   "audio_buffer_rows": w.audio_len, "parallelism": "none (1 GPU)",
                 "schedule": "overlap" if args.overlap else "sequential",
                 "inputs": "distinct per kind" if args.distinct else "two stream triples",
                 "output_gate": bool(args.gated),
                 "qk_prologue": bool(args.qknorm_rope),
                 "flush_mib_between_calls": args.flush_mib},
        "kinds": kinds,
        "roofline": {"kernel": video_kernel_name(w),
                     "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w),
                     "avg_launch_ms": round(vs_ms, 5)},
    }
    if args.qknorm_rope:
        out["qknorm_rope"] = prologue_comparison(lt, ba, dev, outs, w, dpros, stream, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inputs, w, args.cpu_seconds, 3 * args.cpu_seconds)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
        out["cpu_baseline"]["one_core_value"] = round(out["cpu_baseline"]["one_core_value"], 6)
    print(json.dumps(out), flush=True)
    ba.close()


if __name__ == "__main__":
    main()
