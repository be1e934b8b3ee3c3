"""GPU parity of the FP8 QKV GEMM fused with the cache upkeep
(rtv_qkv_gemm_append): Q columns as bf16, K heads rotated and K, V heads
quantized per (token, head) straight into the ring from the float32 result.

Expected values come from the oracle: the float64 GEMM of the same e4m3
operands, and for K the rotation of those values in float64 by the oracle's
float32 (cos, sin) table at the chunk's positions.  The fused path quantizes
the float32 matrix-core result (no bfloat16 in between), so it is checked
within the e4m3 rounding of the exact value plus the GEMM's error bound
carried through the rotation; and most codes must equal the oracle's
quantization of the exact values (a transposed or misplaced row would make
nearly all differ).  Q columns: within the GEMM bound, and bit-identical to
rtv_gemm_fp8's output for the same operands.
"""
import numpy as np
import pytest
import torch

from oracle import bf16 as obf16
from oracle import e4m3 as oe4m3
from oracle import gemm as ogemm
from oracle import quant as oquant
from oracle import rope as orope
from tests.gpu_helpers import ring_rows
from workloads import get_workload
from workloads.generate import projection_inputs

pytestmark = pytest.mark.gpu


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check_rows(codes, scales, exact, err, what, min_same=0.95):
    """codes [n,H,D], scales [n,H] against exact values [n,H,D] known to within err."""
    s = scales.astype(np.float64)
    amax = np.abs(exact).max(axis=2)
    amax_err = err.max(axis=2)
    s_exact = amax / 448.0
    assert np.all(np.abs(s - s_exact) <= amax_err / 448.0 * 1.001 + 2.0 ** -22 * s_exact + 1e-30), \
        f"{what}: row scales off"
    deq = oe4m3.decode(codes).astype(np.float64) * s[..., None]
    tol = 2.0 ** -4 * (np.abs(exact) + err) + 2.0 ** -10 * s[..., None] + err * 1.001 + 1e-30
    bad = np.abs(deq - exact) > tol
    assert not bad.any(), f"{what}: {bad.sum()} values outside the bound, first at {np.argwhere(bad)[:3].tolist()}"
    n, H, D = exact.shape
    want, _ = oquant.quantize_rows(exact.astype(np.float32).reshape(n * H, D))
    same = np.mean(codes.reshape(n * H, D) == want)
    print(f"  {what}: codes equal to the oracle's quantization of the exact values: {same:.4f}", flush=True)
    assert same >= min_same, f"{what}: only {same:.4f} of the codes match"


def _run(rtv, cache, layer, xc, sx, wc, sw, q_cols, rows, positions, base):
    """One fused call; checks the Q output and the chunk's ring rows at `rows`."""
    c = cache.cfg
    H, D = c.n_kv_heads, c.head_dim
    head_frame = cache.layout(layer).head_frame
    xd, wd = _dev(xc), _dev(wc)
    sxd, swd = _dev(np.array([sx], np.float32)), _dev(np.array([sw], np.float32))
    q = rtv.qkv_gemm_append(cache, layer, xd, sxd, wd, swd, q_cols)
    plain = rtv.gemm_fp8(xd, sxd, wd[:q_cols].contiguous(), swd) if q_cols else None
    torch.cuda.synchronize()
    exact = ogemm.gemm_fp64(xc[rows], sx, wc.T, sw)                  # [r, N]
    eb = ogemm.error_bound(xc[rows], sx, wc.T, sw) + 2.0 ** -22 * np.abs(exact)
    if q_cols:
        got = obf16.to_f32(q[torch.as_tensor(rows, device="cuda")].view(torch.int16).cpu().numpy()
                           .view(np.uint16)).astype(np.float64)
        eq = exact[:, :q_cols]
        assert np.all(np.abs(got - eq) <= eb[:, :q_cols] + 2.0 ** -8 * (np.abs(eq) + eb[:, :q_cols])), "Q"
        assert torch.equal(q.view(torch.int16), plain.view(torch.int16)), "Q differs from rtv_gemm_fp8"
    r = len(rows)
    gk = exact[:, q_cols:q_cols + H * D].reshape(r, H, D)
    ek = eb[:, q_cols:q_cols + H * D].reshape(r, H, D)
    gv = exact[:, q_cols + H * D:].reshape(r, H, D)
    ev = eb[:, q_cols + H * D:].reshape(r, H, D)
    cs, sn = orope.cos_sin_table(positions[rows], D, base)
    co = cs.astype(np.float64)[:, None, :]
    si = sn.astype(np.float64)[:, None, :]
    x0, x1 = gk[..., : D // 2], gk[..., D // 2:]
    e0, e1 = ek[..., : D // 2], ek[..., D // 2:]
    rk = np.concatenate([x0 * co - x1 * si, x1 * co + x0 * si], axis=2)
    # float32 products and sum/difference: 3 roundings of 2^-24 relative each
    rnd = 2.0 ** -22 * (np.abs(x0 * co) + np.abs(x1 * si))
    rnd1 = 2.0 ** -22 * (np.abs(x1 * co) + np.abs(x0 * si))
    erk = np.concatenate([np.abs(co) * e0 + np.abs(si) * e1 + rnd, np.abs(co) * e1 + np.abs(si) * e0 + rnd1], axis=2)
    slots = head_frame * c.tokens_per_frame + rows
    kc, ks, vc, vs = ring_rows(cache, layer, slots)
    _check_rows(kc, ks, rk, erk, "K")
    _check_rows(vc, vs, gv, ev, "V")


@pytest.mark.parametrize("T,F,C,D,H,Hq,K", [
    (96, 4, 8, 128, 2, 2, 512),    # 384-token chunks: a full and a partial M tile; Q, K, V in separate N tiles
    (96, 4, 8, 64, 2, 4, 256),     # head_dim 64: K and V heads share an N tile
])
def test_fused_small(rtv_lib, T, F, C, D, H, Hq, K):
    """Three chunks (different ring positions), every token checked."""
    cfg = rtv_lib.RtvConfig(1, Hq, H, D, T, F, C, 8 * F)
    cache = rtv_lib.RtvCache(cfg)
    n = F * T
    q_cols = Hq * D
    N = q_cols + 2 * H * D
    for step in range(3):
        print(f"fused D={D} step={step}", flush=True)
        rng = np.random.default_rng([7, D, step])
        x = rng.standard_normal((n, K), dtype=np.float32)
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / np.sqrt(K))
        xc, sx = ogemm.quantize_per_tensor(x)
        wc, sw = ogemm.quantize_per_tensor(w)
        g0 = cache.layout(0).next_global_frame
        positions = orope.chunk_positions(g0, F, T)
        _run(rtv_lib, cache, 0, xc, sx, wc, sw, q_cols, np.arange(n), positions, cfg.rope_base)
        cache.advance(0)


def test_fused_projection_size_sampled(rtv_lib):
    """X [11968 x 6144], Wt [4608 x 6144] (12 Q + 12 K + 12 V heads of 128):
    the workload's projection fused with the append, sampled tokens checked."""
    wl = get_workload("proj")
    x, w = projection_inputs(wl)
    xc, sx = ogemm.quantize_per_tensor(obf16.to_f32(x))
    wc, sw = ogemm.quantize_per_tensor(obf16.to_f32(np.ascontiguousarray(w.T)))
    H, D = wl.n_kv_heads, wl.head_dim
    q_cols = wl.proj_width - 2 * H * D
    cfg = rtv_lib.RtvConfig(1, wl.n_q_heads, H, D, wl.tokens_per_frame, wl.chunk_frames,
                            wl.capacity_frames, 4 * wl.chunk_frames, wl.rope_base)
    cache = rtv_lib.RtvCache(cfg)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 255, 256, wl.chunk_tokens - 1],
                                     rng.integers(0, wl.chunk_tokens, 12)]))
    positions = orope.chunk_positions(0, wl.chunk_frames, wl.tokens_per_frame)
    print("fused projection size", flush=True)
    _run(rtv_lib, cache, 0, xc, sx, wc, sw, q_cols, rows, positions, cfg.rope_base)


def test_fused_argument_errors(rtv_lib):
    """Shapes the fused projection rejects before enqueuing anything."""
    wl = get_workload("tiny")
    cfg = rtv_lib.RtvConfig(1, 2, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame, wl.chunk_frames,
                            wl.capacity_frames, 2 * wl.chunk_frames)
    c = rtv_lib.RtvCache(cfg)
    abi = rtv_lib.abi
    n, D, H = wl.chunk_tokens, wl.head_dim, wl.n_kv_heads
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    kv = 2 * H * D

    def call(n_tok, k_dim, q_cols, q_ptr=None):
        x = torch.zeros((max(n_tok, 1), k_dim), dtype=torch.uint8, device="cuda")
        w = torch.zeros((q_cols + kv, k_dim), dtype=torch.uint8, device="cuda")
        q = torch.empty((max(n_tok, 1), max(q_cols, 8)), dtype=torch.bfloat16, device="cuda")
        abi.rtv_qkv_gemm_append(c.handle, 0, x.data_ptr(), one.data_ptr(), w.data_ptr(), one.data_ptr(),
                                n_tok, k_dim, q_cols, q.data_ptr() if q_ptr is None else q_ptr, q.stride(0), 0)

    for args, status in (((n - 1, 64, 0), abi.RTV_ERR_INVALID_ARG),      # not one chunk
                         ((n, 60, 0), abi.RTV_ERR_INVALID_ARG),          # k_dim not a multiple of 64
                         ((n, 64, D + 1), abi.RTV_ERR_INVALID_ARG)):     # Q columns not whole heads
        with pytest.raises(rtv_lib.RtvError) as e:
            call(*args)
        assert e.value.status == status, args
    with pytest.raises(rtv_lib.RtvError) as e:
        call(n, 64, D, q_ptr=0)                                          # Q columns without an output
    assert e.value.status == abi.RTV_ERR_INVALID_ARG
    assert c.layout(0).appended == 0
    call(n, 64, 0)                                                      # valid: counts as the append
    c.advance(0)
    call(n, 64, 0)
    c.advance(0)
    with pytest.raises(rtv_lib.RtvError) as e:                          # RoPE table holds 2 chunks
        call(n, 64, 0)
    assert e.value.status == abi.RTV_ERR_STATE
