#!/usr/bin/env python3
"""Decode weight-stream benchmark on one MI355X.

One step = one whole decode frame (every hot-path stage): 36-layer
Qwen3-8B-shaped body (per layer: RMSNorm+QKV, identity attention stub + O +
residual, RMSNorm + gate/up + SwiGLU, down + residual), final RMSNorm + sliced
lm_head over the 16384 reachable rows, Philox Gumbel-argmax draw, depth-decoder
input projection, 7 codebook steps of the 4-layer depth decoder (int8 groups
of 128) each with its head and draw, and the frame-embedding feedback.  The
frame is replayed as a HIP graph; weights are seeded synthetic values already
resident in HBM.

value = algorithmic weight bytes per frame x frames/s (GB/s).  The headline
workload is preset A (bf16 body and lm_head, int8-g128 depth) at B = 1.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode weight-stream GB/s (% of HBM peak) and frames/s at B=1/6/16"
HBM_PEAK_GBS = 8000.0
# Counter-derived HBM bytes of the dominant kernel; valid only for the kernel
# sources it was measured on (their sha256 is recorded beside the figures).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_gate_up_bf16_B1.txt")
KERNEL_SOURCES = ("gemv.hip", "m3_internal.h", "m3_sampling.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_model(preset: str, seed: int, dev: str, keep_layer0: bool = False):
    import torch
    from autoregressive_audio_lm_amd import configs, runtime, synth
    cfg = configs.config("frame-full")
    p = configs.PRESETS[preset]
    t0 = time.time()
    md = synth.make_model(cfg, **p, seed=seed, device=dev)
    host_layer0 = None
    if keep_layer0:
        L0 = md["layers"][0]
        host_layer0 = {k: (synth.bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy())
                       for k, v in L0.items()}
    dm = runtime.DecodeModel(md, seed=seed, free_sources=True)
    del md
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    log(f"[bench] preset {preset}: weights generated and packed in {time.time() - t0:.1f} s, "
        f"{dm.weight_bytes() / 1e9:.3f} GB per frame")
    return cfg, dm, host_layer0


def time_frames(dm, cfg, B, steps, warmup, stream, seed=0):
    import torch
    from autoregressive_audio_lm_amd import runtime, synth
    x0 = synth.activations(B, cfg["H"], 1000 + seed, device="cuda")
    st = runtime.FrameState(dm, B, x0, frame0=0)
    with torch.cuda.stream(stream):
        st.capture(stream)
        for _ in range(warmup):
            st.replay(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            st.replay(stream)
        e1.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / steps
    return st, ms, wall


def time_frames_persistent(dm, cfg, B, steps, warmup, stream, seed=0):
    """Frames as one cooperative launch each; HIP events on the launch stream."""
    import torch
    from autoregressive_audio_lm_amd import runtime, synth
    x0 = synth.activations(B, cfg["H"], 1000 + seed, device="cuda")
    st = runtime.FrameState(dm, B, x0, frame0=0)
    with torch.cuda.stream(stream):
        st.persistent_create(stream)
        for _ in range(warmup):
            st.persistent_launch(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            st.persistent_launch(stream)
        e1.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    if int(st.err.item()) != 0:
        raise RuntimeError("a persistent frame gave up waiting")
    ms = e0.elapsed_time(e1) / steps
    return st, ms, wall


def time_gate_up(dm, st, stream, reps=3):
    """Average duration of the body's gate/up GEMV (RMSNorm prologue + SwiGLU
    epilogue), the frame's dominant kernel, over every layer's matrix, with
    HIP events on the stream the launches go to."""
    import torch
    from autoregressive_audio_lm_amd import m3
    c = dm.config
    H, F = c.hidden, c.ffn
    h = st.h
    mlp = st.view("mlp", torch.bfloat16, F)
    fmt = dm.fmt_body
    with torch.cuda.stream(stream):
        for L in dm.packed_layers[:2]:          # warm the launch path
            m3.gemv(fmt, L["gate_up"], 2 * F, H, h, gamma=L["ffn_norm"], eps=c.eps,
                    y=mlp, epi=m3.EPI_SWIGLU, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n = 0
        for _ in range(reps):
            for L in dm.packed_layers:
                m3.gemv(fmt, L["gate_up"], 2 * F, H, h, gamma=L["ffn_norm"], eps=c.eps,
                        y=mlp, epi=m3.EPI_SWIGLU, stream=stream)
                n += 1
        e1.record(stream)
        stream.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    if fmt == 0:
        wbytes = 2 * (2 * F) * H
    elif fmt == 1:
        wbytes = (2 * F) * H + 4 * (2 * F)
    else:
        wbytes = (2 * F) * H + 4 * (2 * F) * (H // 128)
    return us, wbytes + 4 * H, n


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "autoregressive_audio_lm_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the body gate/up GEMV from the committed
    FETCH_SIZE/WRITE_SIZE passes, or None when the kernel sources changed
    since those counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calib_copy(stream, nbytes=256 << 20, reps=3):
    """A plain elementwise copy of known size (nbytes read, nbytes written),
    the yardstick that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    with torch.cuda.stream(stream):
        src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(reps):
            torch.neg(src, out=dst)
        stream.synchronize()
    del src, dst


def cpu_baseline(cfg, L0, target_s: float):
    """The oracle (plain C, float64 sums) on one body layer of the same
    workload at B = 1, repeated to fill about target_s seconds."""
    import numpy as np
    import oracle as O
    H, F = cfg["H"], cfg["F"]
    nq, nkv, hd = cfg["n_heads"] * 128, cfg["n_kv_heads"] * 128, 128
    mats = dict(qkv=O.Matrix(L0["qkv"], O.BF16), o=O.Matrix(L0["o"], O.BF16),
                gu=O.Matrix(O.interleave_gate_up(L0["gate"], L0["up"]), O.BF16),
                down=O.Matrix(L0["down"], O.BF16))
    layer_bytes = sum(O.matrix_bytes(O.BF16, m.N, m.K) for m in mats.values()) + 2 * 4 * H
    rng = np.random.default_rng(0)
    x = O.f64_to_bf16(rng.standard_normal((1, H)))

    def one_layer(h):
        a = O.rmsnorm(h, L0["attn_norm"], cfg["eps"])
        qkv = O.f64_to_bf16(O.gemv(mats["qkv"], a))
        o = O.attn_stub(qkv, nq + nkv, cfg["n_heads"], cfg["n_heads"] // cfg["n_kv_heads"], hd)
        h = O.residual(O.gemv(mats["o"], o), h)
        a = O.rmsnorm(h, L0["ffn_norm"], cfg["eps"])
        m = O.swiglu_interleaved(O.gemv(mats["gu"], a))
        return O.residual(O.gemv(mats["down"], m), h)

    t0 = time.perf_counter()
    h = one_layer(x)
    t1 = time.perf_counter() - t0
    reps = max(1, min(20000, int(math.ceil(target_s / max(t1, 1e-3))) - 1))
    t0 = time.perf_counter()
    for _ in range(reps):
        h = one_layer(h)
    dt = time.perf_counter() - t0
    return {"value": round(reps * layer_bytes / dt / 1e9, 3), "unit": "GB/s",
            "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{reps} passes of one body layer (bf16 QKV+O+gate/up+down with norms, stub, "
                      f"SwiGLU and residuals; {layer_bytes / 1e6:.1f} MB of weights) at B=1, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--B", type=int, default=1)
    ap.add_argument("--preset", default="A", choices=["A", "B"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true", help="skip the B = 2/6/16 and int8 context points")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 256 MiB elementwise copy (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the decode hot path here runs on a single GPU "
              "(independent songs would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from autoregressive_audio_lm_amd import _lib
    _lib.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    props = torch.cuda.get_device_properties(0)
    stream = torch.cuda.Stream()

    cfg, dm, L0 = build_model(args.preset, args.seed, dev, keep_layer0=not args.no_cpu_baseline)
    fbytes = dm.weight_bytes()
    st, ms, wall = time_frames(dm, cfg, args.B, args.steps, args.warmup, stream, args.seed)
    fps = 1e3 / ms
    gbs = fbytes * fps / 1e9
    log(f"[bench] preset {args.preset} B={args.B}: {ms:.4f} ms/frame, {fps:.1f} frames/s, "
        f"{gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s); wall {wall:.3f} s")

    us, kbytes, n = time_gate_up(dm, st, stream)
    k_gbs = kbytes / (us * 1e-6) / 1e9
    log(f"[bench] gate/up GEMV: {us:.2f} us per launch over {n} launches, {k_gbs:.1f} GB/s")
    traffic = measured_traffic() if (args.preset == "A" and args.B == 1) else None
    roofline = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_kernel<bf16, VALU, SwiGLU> (body gate/up, RMSNorm fused)"
                          if dm.fmt_body == 0 else "gemv_kernel<int8, SwiGLU> (body gate/up)",
                "avg_us": round(us, 3), "bytes_per_launch": kbytes}
    st.release()
    if args.calib_copy:
        calib_copy(stream)

    sweep = []
    if not args.no_sweep:
        for B in (2, 6, 16):
            s2, ms2, _ = time_frames(dm, cfg, B, max(20, args.steps // 4), 3, stream, args.seed)
            s2.release()
            sweep.append({"preset": args.preset, "B": B, "ms_per_frame": round(ms2, 4),
                          "frames_per_s": round(1e3 / ms2, 2),
                          "GB_s": round(fbytes * 1e3 / ms2 / 1e9, 1),
                          "frac_of_hbm_peak": round(fbytes * 1e3 / ms2 / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] sweep {sweep[-1]}")
        other = "B" if args.preset == "A" else "A"
        del st, dm
        torch.cuda.empty_cache()
        _, dm2, _ = build_model(other, args.seed, dev)
        fb2 = dm2.weight_bytes()
        for B in (1, 6, 16):
            s2, ms2, _ = time_frames(dm2, cfg, B, max(20, args.steps // 4), 3, stream, args.seed)
            s2.release()
            sweep.append({"preset": other, "B": B, "bytes_per_frame": fb2,
                          "ms_per_frame": round(ms2, 4), "frames_per_s": round(1e3 / ms2, 2),
                          "GB_s": round(fb2 * 1e3 / ms2 / 1e9, 1),
                          "frac_of_hbm_peak": round(fb2 * 1e3 / ms2 / 1e9 / HBM_PEAK_GBS, 4)})
            log(f"[bench] sweep {sweep[-1]}")
        del dm2
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(cfg, L0, args.cpu_seconds)
        log(f"[bench] cpu_baseline {cpu}")

    fmt_name = {0: "bf16", 1: "int8 per-row", 2: "int8 per-group-128"}
    p = __import__("autoregressive_audio_lm_amd.configs", fromlist=["PRESETS"]).PRESETS[args.preset]
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p["fmt_body"] == 0 else "int8xbf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) input rows; no checkpoint)",
        "config": {
            "workload": (f"one decode frame, preset {args.preset}: 36-layer Qwen3-8B-shaped body "
                         f"({fmt_name[p['fmt_body']]}), sliced lm_head [16384,4096] "
                         f"({fmt_name[p['fmt_lm']]}) + Philox Gumbel-argmax, depth decoder 4 layers "
                         f"x 7 codebooks ({fmt_name[p['fmt_depth']]}) + 7 draws, frame feedback; "
                         f"attention stubbed as identity"),
            "B": args.B,
            "bytes_per_frame": fbytes,
            "graph": "one HIP graph per frame, replayed",
        },
        "frames_per_s": round(fps, 2),
        "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "gpu": f"{props.name} {props.gcnArchName} x{props.multi_processor_count} CU",
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
