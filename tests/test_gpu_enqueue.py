"""The calls of a step only enqueue work (GPU).

A single read-back of device memory per step is reported to have raised the
step time from 168.5 ms to 278 ms (page "Runway explains how it serves a 57B
video model in real time", fifth paragraph), so append, attend and advance in
the host-state mode must neither synchronize nor copy to the host nor
allocate.  Here a step of the full-window layer shape (12 heads x 128, 11968
tokens per chunk, 47872-key window) over 8 layers x 4 (append, attend) calls
and one advance is enqueued from Python: the host must get control back while
the GPU is still busy with the step (the stream is not idle right after the
last call), and the host time of the enqueue must be a small fraction of the
GPU time of the step.  A call that synchronized would make the first check
fail; one that waited on the GPU in any other way would make its host time
grow towards the GPU time.  Both ring-state modes: host state, and device
state (the mode a captured step runs in, where the calls read and move the
ring state in their kernels).
"""
import time

import pytest
import torch

from workloads import get_workload
from workloads.generate import device_normal_bf16

pytestmark = pytest.mark.gpu

N_LAYERS = 8
CALLS = 4


@pytest.mark.parametrize("device_state", [False, True])
def test_step_calls_only_enqueue(rtv_lib, device_state):
    rtv = rtv_lib
    wl = get_workload("step")
    dev = torch.device("cuda:0")
    steps = wl.capacity_frames // wl.chunk_frames + 4
    cfg = rtv.RtvConfig(N_LAYERS, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame,
                        wl.chunk_frames, wl.capacity_frames, (steps + 1) * wl.chunk_frames, wl.rope_base)
    cache = rtv.RtvCache(cfg, device=dev)
    n, H, Hq, D = wl.chunk_tokens, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    inputs = [tuple(device_normal_bf16((n, h, D), (9, layer, t), dev) for t, h in ((0, Hq), (1, H), (2, H)))
              for layer in range(N_LAYERS)]
    out = torch.empty((n, Hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        for _ in range(CALLS):
            for layer in range(N_LAYERS):
                q, k, v = inputs[layer]
                cache.append(layer, k, v, stream=stream)
                cache.attend(layer, q, out, stream=stream)
        cache.advance(-1, stream=stream)

    # fill the rings (every later attend sees the full 16-frame window)
    print(f"enqueue: filling {N_LAYERS} layers", flush=True)
    for _ in range(wl.capacity_frames // wl.chunk_frames):
        step()
    torch.cuda.synchronize()
    assert cache.window(0).window_frames == wl.capacity_frames
    if device_state:
        cache.device_state_begin(stream=stream)    # (synchronizes, once)

    results = []
    for rep in range(3):
        print(f"enqueue: device_state={device_state} timed step {rep}", flush=True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        t0 = time.perf_counter()
        step()
        t1 = time.perf_counter()
        busy = not stream.query()
        e1.record(stream)
        torch.cuda.synchronize()
        gpu_s = e0.elapsed_time(e1) * 1e-3
        results.append((t1 - t0, gpu_s, busy))
        print(f"  host enqueue {1e3 * (t1 - t0):.3f} ms, GPU {1e3 * gpu_s:.3f} ms, "
              f"stream busy after the last call: {busy}")
    if device_state:
        cache.device_state_end(stream=stream)
    for host_s, gpu_s, busy in results:
        assert busy, "the stream was idle when the calls returned: a call waited for the GPU"
        assert host_s < 0.25 * gpu_s, (host_s, gpu_s)
    cache.close()
