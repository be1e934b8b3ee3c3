"""Device-resident ring state and graph capture (rtv_device_state_begin / _end).

In the device-state mode the append, attend and advance calls read and move
the per-layer ring state in their kernels.  Their results must equal the
host-state calls' bit for bit (same kernels, same arithmetic), both when the
calls run eagerly and when a step captured once in a HIP graph is replayed
step after step with new inputs.  Every replay is checked against an eager
host-state run of the same inputs, with eager work and synchronizations
between the replays.
"""
import numpy as np
import pytest
import torch

from oracle.cache import OracleKVCache
from tests.attention_check import check_attention
from tests.gpu_helpers import bf16_to_np_f32, to_dev_bf16
from workloads import get_workload, qkv_normal

pytestmark = pytest.mark.gpu


def _cfg(rtv, wl, n_layers, max_global_frames):
    return rtv.RtvConfig(
        n_layers=n_layers, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
        tokens_per_frame=wl.tokens_per_frame, chunk_frames=wl.chunk_frames,
        capacity_frames=wl.capacity_frames, max_global_frames=max_global_frames,
        rope_base=wl.rope_base)


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def _same_rings(x, y, n_layers):
    for layer in range(n_layers):
        for tx, ty in zip(x.ring_tensors(layer), y.ring_tensors(layer)):
            if not _same(tx, ty):
                return False
    return True


def _inputs(wl, n_layers, step, call):
    return [tuple(to_dev_bf16(a) for a in qkv_normal(wl, layer, step, call)) for layer in range(n_layers)]


def test_device_state_eager_equals_host_state(rtv_lib):
    """Tiny shape, 2 layers, 12 chunks through an 8-frame ring (6 wraps), two
    calls per step with capped and full windows: outputs and ring contents
    bit-identical to the host-state calls; the state comes back to the host."""
    wl = get_workload("tiny")
    n_layers = 2
    cfg = _cfg(rtv_lib, wl, n_layers, (wl.steps + 2) * wl.chunk_frames)
    host, dev = rtv_lib.RtvCache(cfg), rtv_lib.RtvCache(cfg)
    dev.device_state_begin()
    for step in range(wl.steps):
        for call in range(2):
            print(f"device-state eager step={step} call={call}", flush=True)
            maxw = 0 if (step + call) % 3 else wl.chunk_frames
            for layer, (q, k, v) in enumerate(_inputs(wl, n_layers, step, call)):
                for c in (host, dev):
                    c.append(layer, k, v)
                a = host.attend(layer, q, max_window_frames=maxw)
                b = dev.attend(layer, q, max_window_frames=maxw)
                assert _same(a, b), (step, call, layer)
        assert _same_rings(host, dev, n_layers), step
        host.advance(-1)
        dev.advance(-1)
    dev.device_state_end()
    for layer in range(n_layers):
        lh, ld = host.layout(layer), dev.layout(layer)
        assert (lh.next_global_frame, lh.committed_frames) == (ld.next_global_frame, ld.committed_frames)


def _graph_replay_case(rtv_lib, wl, n_layers, steps, capture_at, maxw=0, oracle_rows=None):
    """Eager device-state steps up to capture_at, one step captured, then
    replays with each step's inputs copied into the captured buffers; each
    step compared with an eager host-state cache fed the same inputs and, on
    `oracle_rows` (query rows of every head), with the oracle."""
    cfg = _cfg(rtv_lib, wl, n_layers, (steps + 2) * wl.chunk_frames)
    host, dev = rtv_lib.RtvCache(cfg), rtv_lib.RtvCache(cfg)
    ora = None
    if oracle_rows is not None:
        ora = OracleKVCache(n_layers, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame, wl.chunk_frames,
                            wl.capacity_frames, wl.rope_base)
    bufs = [tuple(t.clone() for t in qkv) for qkv in _inputs(wl, n_layers, 0, 0)]
    outs = [torch.empty_like(q) for q, _, _ in bufs]

    def dev_step():
        for layer, (q, k, v) in enumerate(bufs):
            dev.append(layer, k, v)
            dev.attend(layer, q, outs[layer], max_window_frames=maxw)
        dev.advance(-1)

    dev.device_state_begin()
    graph = None
    for step in range(steps):
        new = _inputs(wl, n_layers, step, 0)
        for (q, k, v), (nq, nk, nv) in zip(bufs, new):
            q.copy_(nq); k.copy_(nk); v.copy_(nv)
        if step < capture_at:
            dev_step()
        else:
            if graph is None:
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    with torch.cuda.graph(graph, stream=side):
                        dev_step()
                torch.cuda.current_stream().wait_stream(side)
            print(f"graph replay step={step}", flush=True)
            graph.replay()
        # the eager host-state reference for the same inputs
        want = []
        for layer, (nq, nk, nv) in enumerate(new):
            host.append(layer, nk, nv)
            want.append(host.attend(layer, nq, max_window_frames=maxw))
        torch.cuda.synchronize()
        for layer in range(n_layers):
            assert _same(outs[layer], want[layer]), (step, layer)
        assert _same_rings(host, dev, n_layers), step
        if ora is not None:
            for layer, (q, k, v) in enumerate(qkv_normal(wl, layer, step, 0) for layer in range(n_layers)):
                ora.append(layer, k, v)
                ref = ora.attend(layer, q, max_window_frames=maxw, rows=oracle_rows)
                check_attention(bf16_to_np_f32(outs[layer])[oracle_rows], ref,
                                f"graph replay step={step} layer={layer} window={ora.window_frames(layer, maxw)}")
                ora.advance(layer)
        host.advance(-1)
    dev.device_state_end()
    for layer in range(n_layers):
        lh, ld = host.layout(layer), dev.layout(layer)
        assert (lh.next_global_frame, lh.committed_frames) == (ld.next_global_frame, ld.committed_frames)


def test_graph_replay_tiny_wraps(rtv_lib):
    """Tiny shape, 2 layers: one step captured after 2 eager steps, replayed
    10 times (the window grows, then the ring wraps 5 times)."""
    wl = get_workload("tiny")
    _graph_replay_case(rtv_lib, wl, n_layers=2, steps=12, capture_at=2)


def test_graph_replay_tiny_capped_window(rtv_lib):
    wl = get_workload("tiny")
    _graph_replay_case(rtv_lib, wl, n_layers=1, steps=8, capture_at=0, maxw=wl.chunk_frames)


def test_graph_replay_layer_shape(rtv_lib):
    """12 heads x 128, 16-frame ring: captured at the first step, replayed while
    the window grows 4 -> 16 frames and once more in steady state (47872 keys,
    split tail and combine); every replay also against the oracle on 64
    sampled query rows of every head."""
    wl = get_workload("layer")
    rows = np.unique(np.concatenate([[0, wl.chunk_tokens - 1],
                                     np.random.default_rng(8).choice(wl.chunk_tokens, 64, replace=False)]))
    _graph_replay_case(rtv_lib, wl, n_layers=1, steps=6, capture_at=0, oracle_rows=rows)


def test_device_state_rope_exhaustion(rtv_lib):
    """A chunk past the end of the RoPE table: the kernels write nothing, the
    advance still moves the state, and rtv_device_state_end reports it."""
    wl = get_workload("tiny")
    cfg = _cfg(rtv_lib, wl, 1, 2 * wl.chunk_frames)
    c = rtv_lib.RtvCache(cfg)
    c.device_state_begin()
    for step in range(3):
        (q, k, v), = _inputs(wl, 1, step, 0)
        ring_before = [t.clone() for t in c.ring_tensors(0)]
        out = torch.full_like(q, 7.0)
        c.append(0, k, v)
        c.attend(0, q, out)
        c.advance(0)
        torch.cuda.synchronize()
        if step == 2:
            assert torch.equal(out, torch.full_like(q, 7.0))
            for a, b in zip(ring_before, c.ring_tensors(0)):
                assert _same(a, b)
        else:
            assert not torch.equal(out, torch.full_like(q, 7.0))
    with pytest.raises(rtv_lib.RtvError) as e:
        c.device_state_end()
    assert e.value.status == rtv_lib.abi.RTV_ERR_STATE
    assert c.layout(0).next_global_frame == 3 * wl.chunk_frames
    with pytest.raises(rtv_lib.RtvError) as e:
        c.device_state_end()
    assert e.value.status == rtv_lib.abi.RTV_ERR_STATE


def test_device_state_call_order_errors(rtv_lib):
    """begin twice, end without begin, and the fused projection (host-state
    only) inside the mode are STATE / UNSUPPORTED errors that change nothing."""
    wl = get_workload("tiny")
    cfg = _cfg(rtv_lib, wl, 1, 4 * wl.chunk_frames)
    c = rtv_lib.RtvCache(cfg)
    abi = rtv_lib.abi
    with pytest.raises(rtv_lib.RtvError) as e:
        c.device_state_end()
    assert e.value.status == abi.RTV_ERR_STATE
    c.device_state_begin()
    with pytest.raises(rtv_lib.RtvError) as e:
        c.device_state_begin()
    assert e.value.status == abi.RTV_ERR_STATE
    n = wl.chunk_tokens
    x = torch.zeros((n, 64), dtype=torch.uint8, device="cuda")
    cols = 2 * wl.n_kv_heads * wl.head_dim
    w = torch.zeros((cols, 64), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(rtv_lib.RtvError) as e:
        rtv_lib.qkv_gemm_append(c, 0, x, one, w, one, 0)
    assert e.value.status == abi.RTV_ERR_UNSUPPORTED
    c.device_state_end()
    assert c.layout(0).next_global_frame == 0
