"""Window-length and head-position sweep, and the hot path's device memory.

The pages report a production failure of a tuned kernel whose tests did not
cover the variety of lengths it met (page "Runway: Πώς ένα AI 57 δισ.
παραμέτρων παράγει βίντεο στα 24 fps", section "Η ποιότητα της εικόνας και τα
προβλήματα της πραγματικής λειτουργίας").  Here every valid window length is
attended at every head position of the ring, for tile-aligned and ragged
chunk sizes, on short rings (windows of 192 to 2304 keys) and on rings whose
windows cross 8192 keys (4000 to 16384 keys, where the one-code kernel and its
peaked-row check take over), with each choice of attention weights:
  - attention against the oracle (the contract's bounds and the relative
    ones), and the ring read back bit for bit for every window;
  - the device-state mode, fed the same calls, bit-identical to the host-state
    mode;
  - a second full pass of the sweep leaves the device's used memory outside
    torch's own pool unchanged (within 1 MiB of runtime noise): the calls
    allocate no device memory.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle.cache import OracleKVCache
from tests.attention_check import check_attention
from tests.gpu_helpers import bf16_to_np_f32, ring_rows, to_dev_bf16
from workloads import get_workload, qkv_normal

pytestmark = pytest.mark.gpu


def _library_bytes() -> int:
    """Device memory in use beyond torch's caching pool."""
    free, total = torch.cuda.mem_get_info()
    return total - free - torch.cuda.memory_reserved()


@pytest.mark.parametrize("T,F,C,D,H,Hq,prob_terms,n_rows", [
    (96, 4, 24, 128, 2, 4, 0, 0),       # 384-token chunks (whole 64-slot tiles), GQA group 2
    (100, 2, 12, 64, 2, 2, 0, 0),       # 200-token chunks: ragged tiles, masked window edges
    (1024, 4, 16, 128, 2, 4, 0, 64),    # windows of 4096 .. 16384 keys, across 8192
    (1024, 4, 16, 128, 2, 4, 1, 64),
    (1024, 4, 16, 128, 2, 4, 2, 64),
    (1000, 4, 16, 128, 2, 2, 0, 64),    # ragged tiles on windows across 8192 keys
    (1000, 4, 16, 128, 2, 2, 2, 64),
])
def test_every_window_at_every_head_position(rtv_lib, T, F, C, D, H, Hq, prob_terms, n_rows):
    """n_rows: query rows checked against the oracle (0 = all).  prob_terms 1
    selects the variant by window length in the host-state mode and by the
    chunk length in the device-state mode, so for it the device-state outputs
    are checked against the oracle instead of bit for bit."""
    wl = dataclasses.replace(get_workload("tiny"), grid_h=1, grid_w=T, chunk_frames=F,
                             capacity_frames=C, head_dim=D, n_kv_heads=H, n_q_heads=Hq)
    positions = C // F
    steps = 2 * positions                      # the ring fills, then every head position occurs
    windows = list(range(F, C + 1, F))
    cfg = rtv_lib.RtvConfig(1, Hq, H, D, T, F, C, (2 * steps + 2) * F, wl.rope_base, prob_terms=prob_terms)
    n = F * T
    rows = (np.arange(n) if n_rows == 0 else
            np.unique(np.concatenate([[0, n - 1], np.random.default_rng(T).choice(n, n_rows, replace=False)])))
    host, dev = rtv_lib.RtvCache(cfg), rtv_lib.RtvCache(cfg)
    ora = OracleKVCache(1, H, D, T, F, C, wl.rope_base)
    dev.device_state_begin()
    n = wl.chunk_tokens
    out_h = torch.empty((n, Hq, D), dtype=torch.bfloat16, device="cuda")
    out_d = torch.empty_like(out_h)
    seen = set()

    def one_pass(check):
        for step in range(steps):
            q, k, v = qkv_normal(wl, 0, step, 0)
            qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
            host.append(0, kd, vd)
            dev.append(0, kd, vd)
            if check:
                ora.append(0, k, v)
            head = host.layout(0).head_frame
            for maxw in windows:
                host.attend(0, qd, out_h, max_window_frames=maxw)
                dev.attend(0, qd, out_d, max_window_frames=maxw)
                if not check:
                    continue
                label = f"sweep T={T} prob_terms={prob_terms} step={step} head={head} window={maxw}"
                print(label, flush=True)
                want = ora.attend(0, q, max_window_frames=maxw, rows=rows)
                check_attention(bf16_to_np_f32(out_h)[rows], want, label)
                if prob_terms == 1 and maxw * T >= 8192:
                    check_attention(bf16_to_np_f32(out_d)[rows], want, label + " device-state")
                else:
                    assert torch.equal(out_h.view(torch.int16), out_d.view(torch.int16)), (step, maxw)
                # the window's tokens at their slots, bit for bit
                frames, tok, kc, ks, vc, vs = ora.window(0, maxw)
                slots = ora.expected_slots(0, maxw)
                gk, gks, gv, gvs = ring_rows(host, 0, slots)
                assert np.array_equal(gk, kc) and np.array_equal(gv, vc)
                assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32))
                assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32))
                w = host.window(0, maxw)
                seen.add((head, w.window_frames))
            host.advance(0)
            dev.advance(0)
            if check:
                ora.advance(0)

    one_pass(check=True)
    # every (head position, window) pair of the steady state occurred
    assert all((h * F, wf) in seen for h in range(positions) for wf in windows), sorted(seen)
    torch.cuda.synchronize()
    before = _library_bytes()
    one_pass(check=False)
    torch.cuda.synchronize()
    grown = _library_bytes() - before
    assert grown <= 1 << 20, f"device memory in use grew by {grown} bytes over a pass of calls"
    dev.device_state_end()
    assert host.layout(0).next_global_frame == dev.layout(0).next_global_frame
