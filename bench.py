"""Benchmark of the cache-upkeep + chunk-attention step on one MI355X.

One step = the per-step hot path at one GPU's head share: for each of 4 calls,
for each of 60 layers, append the 4-frame chunk's K/V (RoPE + e4m3 into the
ring) and attend the chunk's queries over the valid window; then advance every
layer's ring (240 append+attend calls per step, the call count the pages give
for one diffusion step: page "Runway: Πώς ένα AI 57 δισ. παραμέτρων παράγει
βίντεο στα 24 fps", section "Από οκτώ H100 σε τέσσερις").  Shape: 12 KV heads x
128, 2992 tokens per frame (44x68 latent grid), 11968-token chunks, 16-frame
ring (47872 slots).  Inputs are synthetic N(0,1) bf16 drawn on the device, one
(Q, K, V) set per layer, resident in HBM before timing starts.

Prints ONE JSON line (see --help).  The oracle leg (cpu_baseline) times the CPU
oracle on a bounded sample of the same workload and scales it to one step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 matrix peak, TFLOP/s


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--layers", type=int, default=60)
    p.add_argument("--calls", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the timed steps, copy MIB MiB device-to-device once (a kernel of "
                        "known traffic to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="HBM bytes per launch from rocprofv3 counters (optional)")
    return p.parse_args()


def algorithmic(wl, window_frames):
    """Bytes an append must move and flops an attend must compute."""
    n, H, D = wl.chunk_tokens, wl.n_kv_heads, wl.head_dim
    append_bytes = 2 * n * H * D * 2 + 2 * n * H * D + 2 * n * H * 4
    lk = window_frames * wl.tokens_per_frame
    attend_flops = 4.0 * n * lk * D * wl.n_q_heads
    return append_bytes, attend_flops


def cpu_baseline(wl):
    """Time the oracle on a bounded sample and scale it to one step."""
    import numpy as np

    from oracle import attention, bf16, quant, rope
    from workloads import qkv_normal

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    q, k, v = qkv_normal(wl, 0, 0, 0)
    T, F, C = wl.tokens_per_frame, wl.chunk_frames, wl.capacity_frames
    # (a) cache upkeep for one frame's tokens (all heads), x F frames per call
    t0 = time.perf_counter()
    pos = np.arange(12 * T, 13 * T)
    c, s = rope.cos_sin_table(pos, wl.head_dim, wl.rope_base)
    kr = rope.apply_rope(bf16.to_f32(k[:T]), c, s)
    kc, ks = quant.quantize_rows(kr)
    vc, vs = quant.quantize_rows(bf16.to_f32(v[:T]))
    t_append = (time.perf_counter() - t0) * F
    # (b) attention: 128 query rows of one head over a full window of C*T keys
    rng = np.random.default_rng(1)
    kd = quant.dequantize_rows(*quant.quantize_rows(
        rng.standard_normal((C * T, wl.head_dim)).astype(np.float32)))
    vd = quant.dequantize_rows(*quant.quantize_rows(
        rng.standard_normal((C * T, wl.head_dim)).astype(np.float32)))
    rows = 256
    qr = rope.apply_rope(bf16.to_f32(q[:rows, :1]), c[:rows], s[:rows])[:, 0]
    t0 = time.perf_counter()
    attention.attend_rows(qr, kd, vd)
    t_rows = time.perf_counter() - t0
    t_attend = t_rows * (wl.chunk_tokens * wl.n_q_heads / rows)
    step_ms = (t_append + t_attend) * wl.n_layers * wl.calls_per_layer * 1e3
    return {
        "value": round(step_ms, 1), "unit": "ms/step", "cores": int(blas_threads), "kind": "oracle",
        "sample": (f"oracle RoPE+e4m3 upkeep of one frame ({T} tokens x {wl.n_kv_heads} heads) x {F}, "
                   f"and float64 attention of {rows} query rows of one head over {C * T} keys, "
                   f"scaled to {wl.chunk_tokens}x{wl.n_q_heads} rows and "
                   f"{wl.n_layers * wl.calls_per_layer} calls per step"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import dataclasses

    import torch

    import kv_cache_attention_rtv_amd as rtv
    from workloads import get_workload
    from workloads.generate import device_normal_bf16

    wl = dataclasses.replace(get_workload("step"), n_layers=args.layers, calls_per_layer=args.calls)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    total_steps = args.warmup + args.steps
    cfg = rtv.RtvConfig(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                        wl.tokens_per_frame, wl.chunk_frames, wl.capacity_frames,
                        (total_steps + 1) * wl.chunk_frames, wl.rope_base)
    cache = rtv.RtvCache(cfg, device=dev)
    n, H, Hq, D = wl.chunk_tokens, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    inputs = []
    for layer in range(wl.n_layers):
        inputs.append(tuple(device_normal_bf16((n, h, D), (0, layer, t), dev)
                            for t, h in ((0, Hq), (1, H), (2, H))))
    out = torch.empty((n, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def run_step(events=None):
        for call in range(wl.calls_per_layer):
            for layer in range(wl.n_layers):
                q, k, v = inputs[layer]
                if events is not None:
                    events[0].append(torch.cuda.Event(enable_timing=True))
                    events[0][-1].record(stream)
                cache.append(layer, k, v, stream=stream)
                if events is not None:
                    events[1].append(torch.cuda.Event(enable_timing=True))
                    events[1][-1].record(stream)
                cache.attend(layer, q, out, stream=stream)
                if events is not None:
                    events[2].append(torch.cuda.Event(enable_timing=True))
                    events[2][-1].record(stream)
        cache.advance(-1, stream=stream)

    windows = []
    for s in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    ev = ([], [], [])
    step_start = torch.cuda.Event(enable_timing=True)
    step_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_start.record(stream)
    for s in range(args.steps):
        windows.append(cache.window(0).window_frames)
        run_step(ev)
    step_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = step_start.elapsed_time(step_end)
    ms_per_step = gpu_ms / args.steps

    per_call_windows = [w for w in windows for _ in range(wl.calls_per_layer * wl.n_layers)]
    app_ms = [a.elapsed_time(b) for a, b in zip(ev[0], ev[1])]
    att_ms = [a.elapsed_time(b) for a, b in zip(ev[1], ev[2])]
    app_bytes = algorithmic(wl, 0)[0]
    att_flops = [algorithmic(wl, w)[1] for w in per_call_windows]
    att_avg_ms = sum(att_ms) / len(att_ms)
    att_tflops = sum(att_flops) / (sum(att_ms) * 1e-3) / 1e12
    app_avg_ms = sum(app_ms) / len(app_ms)
    app_gbs = app_bytes / (app_avg_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                traffic = json.load(f).get("attend_bytes_per_launch")
        except Exception:
            traffic = None

    result = {
        "metric": "ms/step for 240 append+attend calls (1-GPU head share); HBM GB/s, FP8 MFMA %",
        "value": round(ms_per_step, 3),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (f32 accumulate)",
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.n_layers} layers x {wl.calls_per_layer} (append, attend) calls per step; "
                         f"{H} KV heads x {D}, {Hq} query heads, {wl.tokens_per_frame} tokens/frame, "
                         f"{n}-token chunks, {wl.capacity_frames}-frame ring ({wl.capacity_tokens} slots)"),
            "global_batch": 1, "seq_len": n, "window_frames_timed": sorted(set(windows)),
            "parallelism": "none (one GPU's head share)",
        },
        "roofline": {
            "bound": "mfma", "kernel": "attend_kernel<128>",
            "achieved": round(att_tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(att_tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
            "avg_launch_ms": round(att_avg_ms, 4),
            "flops_per_launch_full_window": algorithmic(wl, wl.capacity_frames)[1],
        },
        "append_roofline": {
            "bound": "hbm", "kernel": "append_rope_quant_kernel<128>",
            "achieved": round(app_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(app_gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(app_avg_ms, 5),
            "bytes_per_launch": app_bytes,
        },
        "wall_s_timed": round(wall, 3),
    }
    if args.copy_calibration:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
