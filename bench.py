"""Benchmark of the cache-upkeep + chunk-attention step on one MI355X.

One step = the per-step hot path at one GPU's head share: for each of 4 calls,
for each of 60 layers, append the 4-frame chunk's K/V (RoPE + e4m3 into the
ring) and attend the chunk's queries over the valid window; then advance every
layer's ring (240 append+attend calls per step, the call count the pages give
for one diffusion step: page "Runway: Πώς ένα AI 57 δισ. παραμέτρων παράγει
βίντεο στα 24 fps", section "Από οκτώ H100 σε τέσσερις").  Shape: 12 KV heads x
128, 2992 tokens per frame (44x68 latent grid), 11968-token chunks, 16-frame
ring (47872 slots).  Inputs are synthetic N(0,1) bf16 drawn on the device, one
(Q, K, V) set per layer, resident in HBM before timing starts.  Every layer's
ring is filled before the warm-up steps, so all timed steps run in the steady
state (full 16-frame window; the four growth steps of a fresh cache are
cheaper and not part of the figure).

By default the timed steps are replays of one HIP graph holding the whole step
(240 appends, 240 attends, the advance), captured once with the ring state in
device memory, as the pages capture the forward pass in a CUDA graph (page
"Runway partage la construction de Runway Characters", fourth paragraph).  The
per-call figures (roofline) come from eagerly launched steps with HIP events
around every call; `--eager` times eager steps for the headline figure too.

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
# the step's attention kernels: the one-code kernel with the peaked-row check,
# and the two-term kernel that recomputes flagged query tiles
ATTEND_KERNEL = "attend16_kernel<false, false, false, true>"
REDO_KERNEL = "attend16_kernel<false, true, true, false>"


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--layers", type=int, default=60)
    p.add_argument("--calls", type=int, default=4)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other workloads' figures (stress ring, GQA, projection) in the default line")
    p.add_argument("--config-steps", type=int, default=10,
                   help="timed calls per figure of the other workloads in the default line")
    p.add_argument("--config-warmup", type=int, default=5,
                   help="untimed calls before each such figure (the clock ramps up after the host-side set-up)")
    p.add_argument("--eager", action="store_true",
                   help="time eagerly launched steps (default: replays of one captured HIP graph per step)")
    p.add_argument("--workload", choices=["step", "projection", "attention"], default="step",
                   help="projection: time the projection workload's chunk (per-tensor e4m3 of X, the FP8 "
                        "QKV GEMM and the append) unfused and fused, one JSON line; attention: one attention "
                        "call at the stress ring's window lengths and at the GQA workload, one JSON line")
    p.add_argument("--no-growth", action="store_true",
                   help="fill the rings with appends only instead of timing the four window-growth steps "
                        "(the profiler runs use it, so that every attention dispatch sees the full window)")
    p.add_argument("--call-steps", type=int, default=2,
                   help="eager steps with HIP events around every call, for the per-call figures")
    p.add_argument("--cpu-heads", type=int, default=8,
                   help="query heads (all chunk rows) the oracle attends in the cpu_baseline sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the timed steps, copy MIB MiB device-to-device once (a kernel of "
                        "known traffic to calibrate rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    p.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                   help="HBM bytes per launch from rocprofv3 counters (optional)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="host only: summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; csv "
                        "output) of this script with --copy-calibration into --traffic-json, then exit")
    p.add_argument("--copy-bytes", type=int, default=1 << 30,
                   help="bytes of the calibration copy in the --pmc runs")
    return p.parse_args()


KERNEL_SOURCES = {
    "attend16_kernel": "kv_cache_attention_rtv_amd/csrc/attend.hip",
    "attend_kernel": "kv_cache_attention_rtv_amd/csrc/attend.hip",
    "combine_kernel": "kv_cache_attention_rtv_amd/csrc/attend.hip",
    "factors_kernel": "kv_cache_attention_rtv_amd/csrc/attend.hip",
    "append_rope_quant_kernel": "kv_cache_attention_rtv_amd/csrc/append.hip",
}


def source_hash(rel: str) -> str:
    import hashlib

    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _kernel_key(name: str):
    import re

    for k in KERNEL_SOURCES:
        if k in name:
            m = re.search(k + r"<[^(]*>", name)
            return m.group(0) if m else k
    if "copyBuffer" in name:
        return "copy"
    return None


def pmc_summary(fetch_dir: str, write_dir: str, copy_bytes: int, out_json: str):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel, scaled by
    what the same counter reads for a device copy of known size."""
    import csv
    import glob

    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no *counter_collection.csv under {d}")
        sums = {}
        for fn in files:
            with open(fn, newline="") as f:
                for row in csv.DictReader(f):
                    if row.get("Counter_Name") != counter:
                        continue
                    key = _kernel_key(row.get("Kernel_Name", ""))
                    if key is None:
                        continue
                    disp = (fn, row.get("Dispatch_Id"))
                    sums.setdefault(key, {}).setdefault(disp, 0.0)
                    sums[key][disp] += float(row["Counter_Value"])
        per[counter] = {k: sum(v.values()) / len(v) for k, v in sums.items()}
        per[counter + "_dispatches"] = {k: len(v) for k, v in sums.items()}
        if "copy" in sums:
            # the calibration copy is the largest copy dispatch of the run (the
            # runtime's small copies use the same kernel)
            per[counter]["copy"] = max(sums["copy"].values())
    calib = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        kib = per[counter].get("copy")
        if not kib:
            raise SystemExit(f"no copy kernel in the {counter} run (run bench.py with --copy-calibration)")
        calib[counter] = copy_bytes / (kib * 1024.0)
    kernels = {}
    for k in per["FETCH_SIZE"]:
        if k == "copy" or k not in per["WRITE_SIZE"]:
            continue
        fb = per["FETCH_SIZE"][k] * 1024.0 * calib["FETCH_SIZE"]
        wb = per["WRITE_SIZE"][k] * 1024.0 * calib["WRITE_SIZE"]
        base = k.split("<")[0]
        kernels[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes": round(fb + wb),
                      "raw_fetch_kib": round(per["FETCH_SIZE"][k], 1),
                      "raw_write_kib": round(per["WRITE_SIZE"][k], 1),
                      "dispatches": per["FETCH_SIZE_dispatches"][k],
                      "source": KERNEL_SOURCES[base], "source_sha256_16": source_hash(KERNEL_SOURCES[base])}
    out = {"calibration": {"copy_bytes": copy_bytes,
                           "fetch_factor": round(calib["FETCH_SIZE"], 4),
                           "write_factor": round(calib["WRITE_SIZE"], 4)},
           "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(out, sort_keys=True))


def traffic_of(path: str, prefix: str):
    """Calibrated HBM bytes per launch of the kernels named `prefix...` in a
    pmc summary, or None when absent or taken from another version of the
    kernel's source."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            kernels = json.load(f)["kernels"]
    except Exception:
        return None
    hits = {k: v for k, v in kernels.items() if k.startswith(prefix)}
    if not hits:
        return None
    for v in hits.values():
        if v.get("source_sha256_16") != source_hash(v["source"]):
            return None
    return hits


def algorithmic(wl, window_frames):
    """Bytes an append must move and flops an attend must compute."""
    n, H, D = wl.chunk_tokens, wl.n_kv_heads, wl.head_dim
    append_bytes = 2 * n * H * D * 2 + 2 * n * H * D + 2 * n * H * 4
    lk = window_frames * wl.tokens_per_frame
    attend_flops = 4.0 * n * lk * D * wl.n_q_heads
    return append_bytes, attend_flops


def cpu_baseline(wl, heads: int):
    """Time the oracle on a bounded sample of one call and scale it to a step:
    the cache upkeep (RoPE + e4m3) of a whole chunk, and float64 attention of
    every query row of `heads` heads (1024-row blocks) over a full window."""
    import numpy as np

    from oracle import attention, bf16, quant, rope
    from workloads import qkv_normal

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = os.cpu_count() or 1
    q, k, v = qkv_normal(wl, 0, 0, 0)
    T, F, C, D = wl.tokens_per_frame, wl.chunk_frames, wl.capacity_frames, wl.head_dim
    n = wl.chunk_tokens
    t0 = time.perf_counter()
    pos = np.arange(C * T, C * T + n)
    c, s = rope.cos_sin_table(pos, D, wl.rope_base)
    quant.quantize_rows(rope.apply_rope(bf16.to_f32(k), c, s))
    quant.quantize_rows(bf16.to_f32(v))
    t_append = time.perf_counter() - t0
    rng = np.random.default_rng(1)
    kd = quant.dequantize_rows(*quant.quantize_rows(rng.standard_normal((C * T, D)).astype(np.float32)))
    vd = quant.dequantize_rows(*quant.quantize_rows(rng.standard_normal((C * T, D)).astype(np.float32)))
    heads = max(1, min(heads, wl.n_q_heads))
    t0 = time.perf_counter()
    for h in range(heads):
        qr = rope.apply_rope(bf16.to_f32(q[:, h:h + 1]), c, s)[:, 0]
        for r0 in range(0, n, 1024):
            attention.attend_rows(qr[r0:r0 + 1024], kd, vd)
    t_heads = time.perf_counter() - t0
    t_attend = t_heads * wl.n_q_heads / heads
    calls = wl.n_layers * wl.calls_per_layer
    step_ms = (t_append + t_attend) * calls * 1e3
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    return {
        "value": round(step_ms, 1), "unit": "ms/step", "cores": int(blas_threads), "kind": "oracle",
        "cpu_count": os.cpu_count(), "affinity_cpus": affinity,
        "sample": (f"one call measured: oracle RoPE+e4m3 upkeep of the {n}-token chunk x {wl.n_kv_heads} "
                   f"heads ({t_append:.2f} s) and float64 attention of all {n} query rows of {heads} of "
                   f"{wl.n_q_heads} heads over {C * T} keys ({t_heads:.2f} s); scaled to {wl.n_q_heads} heads "
                   f"and {calls} calls per step; cores = numpy BLAS threads (elementwise steps use one)"),
    }


def projection(args):
    """The projection workload's chunk: X [11968 x 6144] bf16 to e4m3 (per
    tensor), then either the FP8 GEMM to bf16 QKV [11968 x 4608] followed by
    the append of its K/V columns (unfused), or the GEMM whose epilogue writes
    K/V into the ring (rtv_qkv_gemm_append).  Also one GPU's share of the
    out-projection (quantization and GEMM, O [11968 x 1536] to [11968 x 6144]).
    Inputs N(0,1) (W N(0, 1/K)), drawn on the device."""
    import torch

    import kv_cache_attention_rtv_amd as rtv
    from workloads import get_workload
    from workloads.generate import device_normal_bf16

    wl = get_workload("proj")
    dev = torch.device("cuda:0")
    H, D = wl.n_kv_heads, wl.head_dim
    n, hid, N = wl.chunk_tokens, wl.hidden, wl.proj_width
    q_cols = N - 2 * H * D
    reps = args.steps
    total = 2 * (args.warmup + reps) + 2
    cfg = rtv.RtvConfig(1, wl.n_q_heads, H, D, wl.tokens_per_frame, wl.chunk_frames, wl.capacity_frames,
                        total * wl.chunk_frames, wl.rope_base)
    cache = rtv.RtvCache(cfg, device=dev)
    x = device_normal_bf16((n, hid), (4, 0, 0), dev)
    wt = (device_normal_bf16((N, hid), (4, 0, 1), dev).float() * (1.0 / hid ** 0.5)).to(torch.bfloat16)
    xc, sx = rtv.quant_fp8_per_tensor(x)
    wc, sw = rtv.quant_fp8_per_tensor(wt)
    qkv = torch.empty((n, N), dtype=torch.bfloat16, device=dev)
    q_out = torch.empty((n, q_cols), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rtv.abi.rtv_quant_workspace_bytes(x.numel()), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def quant():
        rtv.quant_fp8_per_tensor(x, xc, sx, ws)

    def gemm():
        rtv.gemm_fp8(xc, sx, wc, sw, qkv)

    def append():
        k = qkv[:, q_cols:q_cols + H * D].unflatten(1, (H, D))
        v = qkv[:, q_cols + H * D:].unflatten(1, (H, D))
        cache.append(0, k, v, stream=stream)
        cache.advance(0, stream=stream)

    def fused():
        rtv.qkv_gemm_append(cache, 0, xc, sx, wc, sw, q_cols, q_out)
        cache.advance(0, stream=stream)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    gemm()
    torch.cuda.synchronize()
    t_quant = timed(quant)
    t_gemm = timed(gemm)
    t_append = timed(append)
    t_fused = timed(fused)
    flops = 2.0 * n * hid * N
    unfused = t_quant + t_gemm + t_append
    result = {
        "metric": "ms per projection chunk (per-tensor e4m3 of X, FP8 QKV GEMM, K/V into the ring)",
        "value": round(t_quant + t_fused, 4), "unit": "ms", "higher_is_better": False,
        "steps": reps, "warmup": args.warmup, "dtype": "fp8-e4m3 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": f"X [{n} x {hid}] bf16, Wt [{N} x {hid}] (Q {q_cols} + K {H * D} + V {H * D} "
                               f"columns), {H} KV heads x {D}, {wl.capacity_frames}-frame ring"},
        "quant_ms": round(t_quant, 4), "gemm_ms": round(t_gemm, 4), "append_ms": round(t_append, 4),
        "unfused_ms": round(unfused, 4), "fused_gemm_append_ms": round(t_fused, 4),
        "fused_ms": round(t_quant + t_fused, 4),
        "gemm_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 1),
        "fused_gemm_tflops": round(flops / (t_fused * 1e-3) / 1e12, 1),
        "gemm_frac_fp8_peak": round(flops / (t_gemm * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "fused_frac_fp8_peak": round(flops / (t_fused * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
    }
    del cache, x, wt, xc, wc, qkv, q_out, ws

    # One GPU's share of the out-projection, the GEMM whose partial sums a
    # tensor-parallel group all-reduces after attention: the attention output
    # of the step's 12 query heads (O [n x 1536] bf16) to e4m3, times Wo^T
    # [6144 x 1536], to a partial [n x 6144] bf16 (the exchange itself needs
    # more than one GPU)
    step_wl = get_workload("step")
    ko = step_wl.n_q_heads * step_wl.head_dim
    o = device_normal_bf16((n, ko), (4, 0, 2), dev)
    wot = (device_normal_bf16((hid, ko), (4, 0, 3), dev).float() * (1.0 / ko ** 0.5)).to(torch.bfloat16)
    oc, so = rtv.quant_fp8_per_tensor(o)
    woc, swo = rtv.quant_fp8_per_tensor(wot)
    part = torch.empty((n, hid), dtype=torch.bfloat16, device=dev)
    ws_o = torch.empty(rtv.abi.rtv_quant_workspace_bytes(o.numel()), dtype=torch.uint8, device=dev)

    def quant_o():
        rtv.quant_fp8_per_tensor(o, oc, so, ws_o)

    def gemm_o():
        rtv.gemm_fp8(oc, so, woc, swo, part)

    t_quant_o = timed(quant_o)
    t_gemm_o = timed(gemm_o)
    flops_o = 2.0 * n * ko * hid
    result["out_projection_share"] = {
        "config": f"O [{n} x {ko}] bf16 ({step_wl.n_q_heads} query heads x {step_wl.head_dim}) to e4m3, "
                  f"times Wo^T [{hid} x {ko}] e4m3, to a partial [{n} x {hid}] bf16 "
                  f"({n * hid * 2 / 1e6:.1f} MB for the all-reduce, not run on one GPU)",
        "quant_ms": round(t_quant_o, 4), "gemm_ms": round(t_gemm_o, 4),
        "gemm_tflops": round(flops_o / (t_gemm_o * 1e-3) / 1e12, 1),
        "gemm_frac_fp8_peak": round(flops_o / (t_gemm_o * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
    }
    del o, wot, oc, woc, part, ws_o
    return result


def attention_configs(args):
    """One attention call at the other configurations the hot path is
    measured on, with the library's default attention weights (one code,
    checked for peaked rows):
    - the stress ring: K/V Student-t (nu = 3) with 4 x20 outlier channels per
      head and 1 % zero rows (the seeded host generator), a 24-frame ring read
      at every window length of its cycle, 4..24 frames (its rows are peaked:
      every query tile is recomputed with two-term queries and weights);
    - the projection workload's attention: 24 query heads over 12 KV heads
      (GQA 2:1) at the full 32-frame ring, 95744 keys (inputs N(0,1) drawn on
      the device);
    - the step's layer shape at the full window with each choice of weights
      (0: checked one code, the default; 1: one code unchecked; 2: two terms).
    Each call is timed between HIP events over `steps` calls after `warmup`."""
    import torch

    import kv_cache_attention_rtv_amd as rtv
    from workloads import get_workload
    from workloads.generate import device_normal_bf16, kv_student_t_outliers

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    def entry(wl, frames, ms):
        keys = frames * wl.tokens_per_frame
        tflops = 4.0 * wl.chunk_tokens * keys * wl.head_dim * wl.n_q_heads / (ms * 1e-3) / 1e12
        return {"window_frames": frames, "keys": keys, "ms": round(ms, 4), "tflops": round(tflops, 1),
                "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4)}

    # the stress ring, filled with its own distribution
    wl = get_workload("stress")
    fills = wl.capacity_frames // wl.chunk_frames
    cfg = rtv.RtvConfig(1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame, wl.chunk_frames,
                        wl.capacity_frames, (fills + 2) * wl.chunk_frames, wl.rope_base)
    cache = rtv.RtvCache(cfg, device=dev)
    def bits_to_dev(bits):
        return torch.from_numpy(bits.view("int16")).view(torch.bfloat16).to(dev)

    for step in range(fills + 1):
        k, v = kv_student_t_outliers(wl, 0, step, 0)
        cache.append(0, bits_to_dev(k), bits_to_dev(v))
        if step < fills:
            cache.advance(0)
    q = device_normal_bf16((wl.chunk_tokens, wl.n_q_heads, wl.head_dim), (5, 0, 0), dev)
    out = torch.empty_like(q)
    stress = []
    for frames in wl.window_cycle:
        ms = timed(lambda: cache.attend(0, q, out, max_window_frames=frames, stream=stream))
        stress.append(dict(entry(wl, frames, ms), recomputed_units=cache.peaked_units()))
    del cache, q, out

    # the projection workload's GQA attention over the full ring
    wp = get_workload("proj")
    fills = wp.capacity_frames // wp.chunk_frames
    cfg = rtv.RtvConfig(1, wp.n_q_heads, wp.n_kv_heads, wp.head_dim, wp.tokens_per_frame, wp.chunk_frames,
                        wp.capacity_frames, (fills + 2) * wp.chunk_frames, wp.rope_base)
    cache = rtv.RtvCache(cfg, device=dev)
    kv_shape = (wp.chunk_tokens, wp.n_kv_heads, wp.head_dim)
    for step in range(fills):
        cache.append(0, device_normal_bf16(kv_shape, (6, step, 1), dev), device_normal_bf16(kv_shape, (6, step, 2), dev))
        if step < fills - 1:
            cache.advance(0)
    q = device_normal_bf16((wp.chunk_tokens, wp.n_q_heads, wp.head_dim), (6, 0, 0), dev)
    out = torch.empty_like(q)
    gqa = entry(wp, wp.capacity_frames, timed(lambda: cache.attend(0, q, out, stream=stream)))
    gqa["recomputed_units"] = cache.peaked_units()
    del cache, q, out

    # the step's layer shape at the full window, with one-code (default) and
    # each choice of attention weights (0: one code checked for peaked rows,
    # the default; 1: one code unchecked; 2: two terms everywhere)
    ws = get_workload("step")
    fills = ws.capacity_frames // ws.chunk_frames
    kv_shape = (ws.chunk_tokens, ws.n_kv_heads, ws.head_dim)
    weights = {}
    for terms in (0, 1, 2):
        cfg = rtv.RtvConfig(1, ws.n_q_heads, ws.n_kv_heads, ws.head_dim, ws.tokens_per_frame, ws.chunk_frames,
                            ws.capacity_frames, (fills + 2) * ws.chunk_frames, ws.rope_base, prob_terms=terms)
        cache = rtv.RtvCache(cfg, device=dev)
        for step in range(fills):
            cache.append(0, device_normal_bf16(kv_shape, (7, step, 1), dev),
                         device_normal_bf16(kv_shape, (7, step, 2), dev))
            if step < fills - 1:
                cache.advance(0)
        q = device_normal_bf16((ws.chunk_tokens, ws.n_q_heads, ws.head_dim), (7, 0, 0), dev)
        out = torch.empty_like(q)
        weights[f"prob_terms_{terms}"] = entry(ws, ws.capacity_frames,
                                               timed(lambda: cache.attend(0, q, out, stream=stream)))
        weights[f"prob_terms_{terms}"]["recomputed_units"] = cache.peaked_units()
        del cache, q, out
    result = {
        "metric": "ms per attention call at the stress ring (every window length) and the GQA workload",
        "value": gqa["ms"], "unit": "ms", "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
        "dtype": "fp8-e4m3 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": (f"stress: {wl.n_q_heads} heads x {wl.head_dim}, {wl.chunk_tokens}-token chunk, "
                                f"Student-t K/V with outlier channels and zero rows, "
                                f"{wl.capacity_frames}-frame ring, windows {list(wl.window_cycle)} frames; "
                                f"gqa: {wp.n_q_heads} query heads over {wp.n_kv_heads} KV heads, "
                                f"{wp.capacity_frames}-frame ring; layer: the step's layer shape at "
                                f"{ws.capacity_frames} frames, prob_terms 0, 1 and 2")},
        "stress": stress, "gqa": gqa, "layer_full_window": weights,
    }
    return result


def main():
    args = parse()
    if args.workload == "attention":
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(attention_configs(args)), flush=True)
        return
    if args.workload == "projection":
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(projection(args)), flush=True)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.copy_bytes, args.traffic_json)
        return
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
    # steps the run makes: ring fill, warm-up, eager steps with per-call
    # events, and (graph mode) one eager device-state step, warm-up replays
    # and the timed replays; the RoPE table covers them all
    total_steps = wl.capacity_frames // wl.chunk_frames + args.warmup + (
        args.steps if args.eager else args.call_steps + 1 + args.warmup + args.steps)
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

    # steady state: fill every layer's ring before the warm-up, so every timed
    # (and warm-up) attend sees the full window.  By default the filling steps
    # are whole steps, timed one by one: the windows of a fresh cache grow
    # 4, 8, 12, 16 frames over them.
    growth = []
    for _ in range(wl.capacity_frames // wl.chunk_frames):
        if args.no_growth:
            for layer in range(wl.n_layers):
                cache.append(layer, inputs[layer][1], inputs[layer][2], stream=stream)
            cache.advance(-1, stream=stream)
            continue
        wf = cache.window(0).window_frames
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run_step()
        b.record(stream)
        growth.append((wf, a, b))
    torch.cuda.synchronize()
    growth = [(wf, a.elapsed_time(b)) for wf, a, b in growth]
    windows = []
    for s in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    def timed(k, body):
        """k steps of body() between HIP events on the stream; (GPU ms, wall s)."""
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        start.record(stream)
        for _ in range(k):
            body()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end), time.perf_counter() - wall0

    # eager steps with an event pair around every call: the per-call figures
    ev = ([], [], [])
    n_call_steps = args.steps if args.eager else args.call_steps

    def eager_step():
        windows.append(cache.window(0).window_frames)
        run_step(ev)
    eager_ms, eager_wall = timed(n_call_steps, eager_step)
    mode = "eager launches"
    per_step = None
    if args.eager:
        gpu_ms, wall = eager_ms, eager_wall
    else:
        # one step captured in a HIP graph with the ring state in device
        # memory; warm-up replays, then the timed replays
        cache.device_state_begin(stream=stream)
        run_step()                            # eager step in the device-state mode
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        torch.cuda.synchronize()
        main_stream = stream
        stream = side
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                run_step()
        stream = main_stream
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        step_events = []

        def replay():
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            graph.replay()
            b.record(stream)
            step_events.append((a, b))
        gpu_ms, wall = timed(args.steps, replay)
        per_step = sorted(a.elapsed_time(b) for a, b in step_events)
        cache.device_state_end(stream=stream)
        windows.append(cache.window(0).window_frames)
        mode = "one HIP graph per step (device-resident ring state), replayed"
    ms_per_step = gpu_ms / args.steps

    per_call_windows = [w for w in windows[:n_call_steps] for _ in range(wl.calls_per_layer * wl.n_layers)]
    app_ms = [a.elapsed_time(b) for a, b in zip(ev[0], ev[1])]
    att_ms = [a.elapsed_time(b) for a, b in zip(ev[1], ev[2])]
    app_bytes = algorithmic(wl, 0)[0]
    att_flops = [algorithmic(wl, w)[1] for w in per_call_windows]
    att_avg_ms = sum(att_ms) / len(att_ms)
    att_tflops = sum(att_flops) / (sum(att_ms) * 1e-3) / 1e12
    app_avg_ms = sum(app_ms) / len(app_ms)
    app_gbs = app_bytes / (app_avg_ms * 1e-3) / 1e9

    # HBM bytes per rtv_attend call (attention + combine kernels of the
    # steady-state window) and per append, from the calibrated counters
    att_traffic = traffic_of(args.traffic_json, ATTEND_KERNEL)
    comb_traffic = traffic_of(args.traffic_json, "combine_kernel<128>")
    fac_traffic = traffic_of(args.traffic_json, "factors_kernel")
    redo_traffic = traffic_of(args.traffic_json, REDO_KERNEL)
    app_traffic = traffic_of(args.traffic_json, "append_rope_quant_kernel<128")
    traffic = None
    if att_traffic:
        traffic = sum(v["bytes"] for v in att_traffic.values())
        for extra in (comb_traffic, fac_traffic, redo_traffic):
            if extra:
                traffic += sum(v["bytes"] for v in extra.values())
    app_bytes_measured = sum(v["bytes"] for v in app_traffic.values()) if app_traffic else None

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
            "parallelism": "none (one GPU's head share)", "launch": mode,
        },
        "eager_ms_per_step": round(eager_ms / n_call_steps, 3),
        "step_ms_median_min": ([round(per_step[len(per_step) // 2], 3), round(per_step[0], 3)]
                               if per_step else None),
        "growth_steps_ms": [{"window_frames": wf, "ms": round(ms, 3)} for wf, ms in growth] or None,
        "tokens_appended_per_s": round(wl.calls_per_layer * wl.n_layers * n / (ms_per_step * 1e-3)),
        "roofline": {
            "bound": "mfma",
            "kernel": (f"rtv_attend = factors_kernel<128> + {ATTEND_KERNEL} + combine_kernel<128> "
                       f"(+ {REDO_KERNEL} and a second combine_kernel<128>, which recompute the query "
                       f"tiles flagged as peaked and exit at once when none is)"),
            "achieved": round(att_tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(att_tflops / FP8_PEAK_TFLOPS, 4), "traffic": traffic,
            "avg_launch_ms": round(att_avg_ms, 4),
            "flops_per_launch_full_window": algorithmic(wl, wl.capacity_frames)[1],
        },
        "append_roofline": {
            "bound": "hbm", "kernel": "append_rope_quant_kernel<128, 3> (3 KV heads per workgroup)",
            "achieved": round(app_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(app_gbs / HBM_PEAK_GBS, 4), "avg_launch_ms": round(app_avg_ms, 5),
            "bytes_per_launch": app_bytes, "traffic": app_bytes_measured,
        },
        "wall_s_timed": round(wall, 3),
        "recomputed_units_last_call": cache.peaked_units(stream=stream),
    }
    # a plain streaming reference for the append's traffic: torch's elementwise
    # add of each layer's K and V into one bf16 tensor reads the same 73.5 MB
    # and writes 36.8 MB (the codes' bytes, without the scales and the RoPE
    # table), one launch per layer on the same cold inputs, events around each
    ref_out = torch.empty_like(inputs[0][1])
    ref_ev = []
    for _ in range(2):
        for layer in range(wl.n_layers):
            a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_ev.record(stream)
            torch.add(inputs[layer][1], inputs[layer][2], out=ref_out)
            b_ev.record(stream)
            ref_ev.append((a_ev, b_ev))
    torch.cuda.synchronize()
    ref_ms = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in ref_ev[wl.n_layers:])
    ref_bytes = 3 * inputs[0][1].numel() * 2
    ref_avg = sum(ref_ms) / len(ref_ms)
    result["append_roofline"]["streaming_reference"] = {
        "kernel": "torch.add(K, V) into bf16 (one elementwise launch per layer, cold inputs)",
        "bytes_per_launch": ref_bytes, "avg_launch_ms": round(ref_avg, 5),
        "median_launch_ms": round(ref_ms[len(ref_ms) // 2], 5),
        "achieved": round(ref_bytes / (ref_avg * 1e-3) / 1e9, 1),
        "frac": round(ref_bytes / (ref_avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "append_time_over_reference": round(app_avg_ms / ref_avg, 3),
        # the two move different bytes: the append's rate over the reference's,
        # counting the append's algorithmic bytes and the chunk's RoPE table
        # rows (n x D floats), which it must read
        "append_rate_over_reference": round(
            ((app_bytes + n * wl.head_dim * 4) / app_avg_ms) / (ref_bytes / ref_avg), 3),
    }
    del ref_out
    if args.copy_calibration:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
    if not args.no_configs:
        # the other workloads' figures, in the same line (parity-test cases,
        # not the headline): the stress ring at every window length, the GQA
        # attention over 95744 keys, the layer shape with each weight choice,
        # and the projection chunk
        del inputs, out
        cache.close()
        del cache
        torch.cuda.empty_cache()
        sub = argparse.Namespace(**vars(args))
        sub.steps, sub.warmup = args.config_steps, args.config_warmup
        att = attention_configs(sub)
        result["configs"] = {"stress_ring": att["stress"], "gqa_95744_keys": att["gqa"],
                             "layer_full_window_by_weights": att["layer_full_window"],
                             "projection_chunk": {k: v for k, v in projection(sub).items()
                                                  if k not in ("metric", "value", "unit", "higher_is_better",
                                                               "steps", "warmup", "data")}}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_heads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
