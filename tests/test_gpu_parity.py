"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bit-exact: e4m3 codes, f32 scales and ring slots.  Attention: max |err| <= 2e-2
and mean |err| <= 2e-3 against float64 attention on the dequantized cache
(N(0,1) workloads); the stress workload is checked normalised by the window's
max |V| (its heavy-tailed V makes absolute errors scale with |V|).
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle.cache import OracleKVCache
from oracle import e4m3 as oe4m3
from tests.gpu_helpers import attention_errors, bf16_to_np_f32, ring_rows, to_dev_bf16, vt_key
from workloads import get_workload, qkv_normal

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def _caches(rtv, wl, max_global_frames=None, n_layers=None, query_terms=1, prob_terms=1):
    steps = max(wl.steps, 1)
    cfg = rtv.RtvConfig(
        n_layers=n_layers or wl.n_layers, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
        head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame, chunk_frames=wl.chunk_frames,
        capacity_frames=wl.capacity_frames,
        max_global_frames=max_global_frames or (steps + 2) * wl.chunk_frames,
        rope_base=wl.rope_base, query_terms=query_terms, prob_terms=prob_terms)
    gpu = rtv.RtvCache(cfg)
    ora = OracleKVCache(cfg.n_layers, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame,
                        wl.chunk_frames, wl.capacity_frames, wl.rope_base)
    return gpu, ora


def _check_ring(gpu, ora, layer, max_window=0):
    """Every window token's codes/scales at its expected slot, bit for bit."""
    frames, tok, kc, ks, vc, vs = ora.window(layer, max_window)
    slots = ora.expected_slots(layer, max_window)
    w = gpu.window(layer, max_window)
    assert w.window_frames == ora.window_frames(layer, max_window)
    seg = np.concatenate([np.arange(w.seg_start[i], w.seg_start[i] + w.seg_len[i])
                          for i in range(w.n_segments)])
    assert np.array_equal(np.sort(seg), np.sort(slots))
    gk, gks, gv, gvs = ring_rows(gpu, layer, slots)
    assert np.array_equal(gk, kc), f"K codes differ at {np.argwhere(gk != kc)[:3].tolist()}"
    assert np.array_equal(gks.view(np.uint32), ks.view(np.uint32)), "K scales differ"
    assert np.array_equal(gv, vc), f"V codes differ at {np.argwhere(gv != vc)[:3].tolist()}"
    assert np.array_equal(gvs.view(np.uint32), vs.view(np.uint32)), "V scales differ"


def test_e4m3_conversion_matches_oracle(rtv_lib):
    top = np.array([464.0], dtype=np.float32).view(np.uint32)[0]
    bits = np.arange(0, top, 61, dtype=np.uint32)
    mids = ((oe4m3.POS_VALUES[:-1] + oe4m3.POS_VALUES[1:]) / 2).astype(np.float32).view(np.uint32)
    near = (mids[:, None].astype(np.int64) + np.arange(-256, 257)[None, :]).ravel().astype(np.uint32)
    vals = oe4m3.POS_VALUES.astype(np.float32).view(np.uint32)
    y = np.concatenate([bits, near, vals]).view(np.float32)
    y = np.concatenate([y, -y, np.array([448.0, 450.0, 463.9, 464.0, 1e9, -0.0], np.float32)])
    y = y[: (len(y) // 4) * 4 + 3]                     # exercise the ragged tail
    x = torch.from_numpy(y).cuda()
    out = torch.empty(len(y), dtype=torch.uint8, device="cuda")
    rtv_lib.abi.rtv_encode_e4m3(x.data_ptr(), out.data_ptr(), len(y),
                                torch.cuda.current_stream().cuda_stream)
    got = out.cpu().numpy()
    want = oe4m3.encode(y)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(y[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("group", [1, 2])
def test_tiny_stream_wraps(rtv_lib, group):
    """12 chunks through an 8-frame ring (6 wraps), two calls per step, head_dim 64."""
    wl = get_workload("tiny")
    if group == 2:
        wl = dataclasses.replace(wl, n_q_heads=4)
    gpu, ora = _caches(rtv_lib, wl)
    worst = (0.0, 0.0)
    for step in range(wl.steps):
        for call in range(2):
            q, k, v = qkv_normal(wl, 0, step, call)
            print(f"tiny group={group} step={step} call={call}", flush=True)
            gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
            ora.append(0, k, v)
            maxw = 0 if (step + call) % 3 else wl.chunk_frames
            out = gpu.attend(0, to_dev_bf16(q), max_window_frames=maxw)
            want = ora.attend(0, q, max_window_frames=maxw)
            mx, mean = attention_errors(bf16_to_np_f32(out), want)
            worst = (max(worst[0], mx), max(worst[1], mean))
            assert mx <= MAX_ABS and mean <= MEAN_ABS, (step, call, mx, mean)
        _check_ring(gpu, ora, 0)
        _check_ring(gpu, ora, 0, wl.chunk_frames)
        gpu.advance(0)
        ora.advance(0)
    print("tiny worst attention error (max, mean):", worst)


def test_poison_outside_window_and_determinism(rtv_lib):
    """NaN codes / scales in every slot outside the window leave the output
    bit-identical; the same call twice gives identical bits."""
    wl = get_workload("tiny")
    gpu, ora = _caches(rtv_lib, wl)
    for step in range(5):
        q, k, v = qkv_normal(wl, 0, step, 0)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        if step < 4:
            gpu.advance(0)
    qd = to_dev_bf16(q)
    for maxw in (4, 8):
        ref = gpu.attend(0, qd, max_window_frames=maxw).clone()
        again = gpu.attend(0, qd, max_window_frames=maxw)
        assert torch.equal(ref.view(torch.int16), again.view(torch.int16))
        w = gpu.window(0, maxw)
        inside = np.zeros(wl.capacity_tokens + 64, dtype=bool)
        for i in range(w.n_segments):
            inside[w.seg_start[i]: w.seg_start[i] + w.seg_len[i]] = True
        kc, vc, ks, vs = gpu.ring_tensors(0)
        saved = [t.clone() for t in (kc, vc, ks, vs)]
        out_slots = torch.as_tensor(np.nonzero(~inside[: kc.shape[1]])[0], device="cuda")
        if out_slots.numel():
            kc[:, out_slots, :] = 0x7F
            ks[:, out_slots] = float("nan")
            vs[:, out_slots] = float("nan")
            pos_of_key = torch.as_tensor(np.argsort(vt_key(np.arange(64))), device="cuda")
            tiles = out_slots // 64
            pos = pos_of_key[out_slots % 64]
            vc[:, tiles, :, pos] = 0x7F
        got = gpu.attend(0, qd, max_window_frames=maxw)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), maxw
        for t, s in zip((kc, vc, ks, vs), saved):
            t.copy_(s)


def test_layer_shape_steady_state(rtv_lib):
    """12 heads x 128, 2992 tokens/frame, 16-frame ring: 5 steps (the window
    grows 4 -> 16 frames and the ring wraps); codes bit-exact every step,
    attention on sampled query rows."""
    wl = get_workload("layer")
    gpu, ora = _caches(rtv_lib, wl, max_global_frames=8 * wl.chunk_frames)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, wl.chunk_tokens - 1],
                                     rng.integers(0, wl.chunk_tokens, 27)]))
    for step in range(5):
        q, k, v = qkv_normal(wl, 0, step, 0)
        print(f"layer step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        e = ora.append(0, k, v)
        L = gpu.layout(0)
        slots = (L.head_frame * wl.tokens_per_frame + np.arange(wl.chunk_tokens))
        gk, gks, gv, gvs = ring_rows(gpu, 0, slots)
        assert np.array_equal(gk, e.k_codes) and np.array_equal(gv, e.v_codes)
        assert np.array_equal(gks.view(np.uint32), e.k_scales.view(np.uint32))
        assert np.array_equal(gvs.view(np.uint32), e.v_scales.view(np.uint32))
        out = gpu.attend(0, to_dev_bf16(q))
        if step in (0, 4):
            want = ora.attend(0, q, rows=rows)
            mx, mean = attention_errors(bf16_to_np_f32(out)[rows], want)
            print(f"layer step={step} attention max={mx:.3e} mean={mean:.3e}", flush=True)
            assert mx <= MAX_ABS and mean <= MEAN_ABS
        gpu.advance(0)
        ora.advance(0)


def test_state_errors(rtv_lib):
    wl = get_workload("tiny")
    gpu, _ = _caches(rtv_lib, wl, max_global_frames=2 * wl.chunk_frames)
    q, k, v = qkv_normal(wl, 0, 0, 0)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    abi = rtv_lib.abi
    with pytest.raises(rtv_lib.RtvError) as e:
        gpu.attend(0, qd)
    assert e.value.status == abi.RTV_ERR_STATE
    with pytest.raises(rtv_lib.RtvError) as e:
        gpu.advance(0)
    assert e.value.status == abi.RTV_ERR_STATE
    with pytest.raises(rtv_lib.RtvError) as e:
        gpu.append(1, kd, vd)
    assert e.value.status == abi.RTV_ERR_INVALID_ARG
    with pytest.raises(rtv_lib.RtvError) as e:
        gpu.append(0, kd[:-1], vd[:-1])
    assert e.value.status == abi.RTV_ERR_INVALID_ARG
    gpu.append(0, kd, vd)
    with pytest.raises(rtv_lib.RtvError) as e:
        gpu.attend(0, qd, max_window_frames=2)
    assert e.value.status == abi.RTV_ERR_INVALID_ARG
    gpu.advance(0)
    gpu.append(0, kd, vd)
    gpu.advance(0)
    with pytest.raises(rtv_lib.RtvError) as e:     # RoPE table holds 2 chunks
        gpu.append(0, kd, vd)
    assert e.value.status == abi.RTV_ERR_STATE
    L = gpu.layout(0)
    assert L.next_global_frame == 2 * wl.chunk_frames and L.appended == 0


@pytest.mark.parametrize("T,F,C,D,H,Hq,steps", [
    (100, 2, 6, 128, 2, 4, 7),      # 200-token chunks: ragged 64-slot tiles, short windows
    (100, 2, 6, 64, 2, 2, 7),
    (2000, 2, 6, 128, 1, 2, 5),     # 4000-token chunks: ragged tiles, windows >= 8192 keys
])
def test_unaligned_chunks(rtv_lib, T, F, C, D, H, Hq, steps):
    """Chunks whose token count is not a multiple of 64: appends write partial
    64-slot tiles and attention masks the ragged tile edges of the window."""
    wl = dataclasses.replace(get_workload("tiny"), grid_h=1, grid_w=T, chunk_frames=F,
                             capacity_frames=C, head_dim=D, n_kv_heads=H, n_q_heads=Hq,
                             steps=steps)
    gpu, ora = _caches(rtv_lib, wl)
    for step in range(steps):
        q, k, v = qkv_normal(wl, 0, step, 0)
        print(f"unaligned T={T} F={F} D={D} step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        ora.append(0, k, v)
        for maxw in (0, F):
            out = gpu.attend(0, to_dev_bf16(q), max_window_frames=maxw)
            want = ora.attend(0, q, max_window_frames=maxw)
            mx, mean = attention_errors(bf16_to_np_f32(out), want)
            assert mx <= MAX_ABS and mean <= MEAN_ABS, (step, maxw, mx, mean)
        _check_ring(gpu, ora, 0)
        gpu.advance(0)
        ora.advance(0)


def test_stress_outliers_zero_rows_window_cycle(rtv_lib):
    """Student-t (nu = 3) K/V with four x20 outlier channels per head and 1 %
    all-zero token rows, a 24-frame ring and a window cycling over 4..24 frames.
    Codes/scales bit-exact (zero rows: scale 0, codes 0x00); attention checked
    normalised by the window's max |V| (heavy tails make absolute errors scale
    with |V|).  The cache carries queries as two e4m3 terms: the outlier
    channels spread the scores over many binades, where one term's rounding
    (2^-4 relative) would move the heaviest keys' weights too far."""
    from workloads.generate import zero_rows
    wl = get_workload("stress")
    gpu, ora = _caches(rtv_lib, wl, max_global_frames=10 * wl.chunk_frames, query_terms=2)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, wl.chunk_tokens - 1], rng.integers(0, wl.chunk_tokens, 30)]))
    cycle = wl.window_cycle
    worst = (0.0, 0.0)
    for step in range(8):
        q, k, v = qkv_normal(wl, 0, step, 0)
        print(f"stress step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        e = ora.append(0, k, v)
        L = gpu.layout(0)
        slots = L.head_frame * wl.tokens_per_frame + np.arange(wl.chunk_tokens)
        gk, gks, gv, gvs = ring_rows(gpu, 0, slots)
        assert np.array_equal(gk, e.k_codes) and np.array_equal(gv, e.v_codes)
        assert np.array_equal(gks.view(np.uint32), e.k_scales.view(np.uint32))
        assert np.array_equal(gvs.view(np.uint32), e.v_scales.view(np.uint32))
        z = zero_rows(wl, 0, step, 0)
        # zero rows: scale 0 and signed-zero codes (RoPE of a zero row may give -0)
        assert np.all(gks[z] == 0) and np.all(gvs[z] == 0)
        assert np.all((gk[z] & 0x7F) == 0) and np.all(gv[z] == 0)
        maxw = cycle[(step + 3) % len(cycle)]
        out = gpu.attend(0, to_dev_bf16(q), max_window_frames=maxw)
        if step >= 4:
            want = ora.attend(0, q, max_window_frames=maxw, rows=rows)
            _, _, _, _, vc, vs = ora.window(0, maxw)
            from oracle import quant
            got = bf16_to_np_f32(out)[rows]
            for h in range(wl.n_q_heads):
                vmax = np.abs(quant.dequantize_rows(vc[:, h], vs[:, h])).max()
                err = np.abs(got[:, h].astype(np.float64) - want[:, h]) / vmax
                worst = (max(worst[0], err.max()), max(worst[1], err.mean()))
                assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (step, maxw, h, err.max(), err.mean())
            print(f"stress step={step} window={maxw} normalised worst so far max={worst[0]:.3e} mean={worst[1]:.3e}", flush=True)
        gpu.advance(0)
        ora.advance(0)


@pytest.mark.parametrize("D,H", [(128, 4), (64, 3)])
def test_append_extreme_row_magnitudes(rtv_lib, D, H):
    """Rows whose magnitudes reach the ends of the float range: scales of
    2^-89 (just inside the short form of the quantization, which needs amax >=
    448 * 2^-100), 2^-93 (either side of that bound), 2^-120, 2^-128 and 2^-133
    (subnormal bf16 values), 2^100 and 2^125 (near the bf16 maximum), all-zero
    rows, and rows of -0.0 with one nonzero value (signed zeros in a row with
    a normal scale).  Per (token, head) classes: in blocks of 8 tokens (one
    wave of the append holds 8 rows) over the first half of the chunk, so that
    whole waves take one form, and at random over the second half, so that
    waves mix them.  Codes and scales bit-exact against the oracle."""
    from workloads.generate import bf16_bits_to_f32, f32_to_bf16_bits
    wl = dataclasses.replace(get_workload("tiny"), head_dim=D, n_kv_heads=H, n_q_heads=H)
    gpu, ora = _caches(rtv_lib, wl, max_global_frames=4 * wl.chunk_frames)
    exps = [0, -89, -93, -120, -128, -133, 100, 125]
    n_cls = len(exps) + 2
    n = wl.chunk_tokens
    for step in range(3):
        _, k, v = qkv_normal(wl, 0, step, 0)
        rng = np.random.default_rng([11, D, step])
        tok = np.arange(n)
        cls_t = np.where(tok < n // 2, (tok // 8) % n_cls, rng.integers(0, n_cls, n))
        cls = (cls_t[:, None] + np.arange(H)[None, :]) % n_cls          # [n, H]

        def shape_rows(bits, salt):
            x = bf16_bits_to_f32(bits).astype(np.float64)
            out = np.zeros_like(x)
            for c, e in enumerate(exps):
                m = cls == c
                out[m] = x[m] * 2.0 ** e
            negz = cls == len(exps) + 1
            out[negz] = -0.0
            ti, hi = np.nonzero(negz)
            out[ti, hi, (ti * 7 + hi + salt) % D] = x[ti, hi, 0]
            return f32_to_bf16_bits(out.astype(np.float32)).reshape(bits.shape)

        k2, v2 = shape_rows(k, 0), shape_rows(v, 3)
        print(f"extreme magnitudes D={D} step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k2), to_dev_bf16(v2))
        e = ora.append(0, k2, v2)
        L = gpu.layout(0)
        slots = L.head_frame * wl.tokens_per_frame + tok
        gk, gks, gv, gvs = ring_rows(gpu, 0, slots)
        for what, got, want in (("K codes", gk, e.k_codes), ("V codes", gv, e.v_codes),
                                ("K scales", gks.view(np.uint32), e.k_scales.view(np.uint32)),
                                ("V scales", gvs.view(np.uint32), e.v_scales.view(np.uint32))):
            bad = np.argwhere(got != want)
            assert bad.size == 0, (what, step, bad[:4].tolist(), [int(cls[t, h]) for t, h, *_ in bad[:4]])
        gpu.advance(0)
        ora.advance(0)


@pytest.mark.parametrize("T", [1024, 96])
def test_attention_rescales_when_later_keys_score_higher(rtv_lib, T):
    """Two chunks whose first 64 keys (the window's first tile) have K scaled
    by 1/4 (exact in bf16): the running max starts from that tile and then has
    to move for most queries during the walk, at different tiles for different
    queries (both query blocks of a lane, the 4-lane reduction and the
    per-lane factor of the rescale), while the softmax over the whole window
    keeps the shape of the N(0,1) workloads.  T = 1024: 8192-key window (codes
    of P' from the log domain); T = 96: 768 keys (two-term P').  12 heads of
    128 over 6 KV heads (GQA 2:1); attention on sampled rows."""
    from oracle import quant
    from workloads.generate import bf16_bits_to_f32, f32_to_bf16_bits
    wl = dataclasses.replace(get_workload("tiny"), grid_h=1, grid_w=T, chunk_frames=4, capacity_frames=8,
                             head_dim=128, n_kv_heads=6, n_q_heads=12)
    gpu, ora = _caches(rtv_lib, wl, max_global_frames=4 * wl.chunk_frames)
    n = wl.chunk_tokens
    rows = np.unique(np.concatenate([[0, 31, 32, 255, 256, n - 1], np.random.default_rng(9).integers(0, n, 26)]))
    for step in range(2):
        q, k, v = qkv_normal(wl, 0, step, 0)
        if step == 0:
            kf = bf16_bits_to_f32(k).reshape(k.shape)
            kf[:64] *= np.float32(0.25)
            k = f32_to_bf16_bits(kf).reshape(k.shape)
        print(f"rescale T={T} step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        ora.append(0, k, v)
        if step == 0:
            gpu.advance(0)
            ora.advance(0)
    # the max does move: for most sampled rows the window's top score is more
    # than 3 octaves above the top score of its first 64 keys (the headroom the
    # running max leaves)
    q_rot = ora.rotated_queries(0, q)
    _, _, kc, ks, _, _ = ora.window(0)
    kd = quant.dequantize_rows(kc[:, 0, :], ks[:, 0])
    s = (q_rot[rows, 0, :].astype(np.float64) @ kd.T) / np.sqrt(128.0) * np.log2(np.e)
    rising = np.mean(s.max(axis=1) - s[:, :64].max(axis=1) > 3.0)
    print(f"rows whose max rises > 3 octaves after the first tile: {rising:.2f}", flush=True)
    assert rising >= 0.5
    out = gpu.attend(0, to_dev_bf16(q))
    want = ora.attend(0, q, rows=rows)
    mx, mean = attention_errors(bf16_to_np_f32(out)[rows], want)
    print(f"rescale T={T} attention max={mx:.3e} mean={mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


@pytest.mark.parametrize("prob_terms", [1, 2])
def test_peaked_attention_and_two_term_weights(rtv_lib, prob_terms):
    """Peaked attention on an 8192-key window: the second chunk's K doubled
    (exact in bf16), so its scores spread twice as wide and a few keys carry
    much of each row's weight.  The one-code weights of long windows (within
    one code step of the rounded value) then no longer average out: their
    error is reported, and the cache created with prob_terms = 2 (exp2 and two
    e4m3 terms per weight) must meet the tolerance.  12 heads of 128 over 6 KV
    heads; attention on sampled rows."""
    from workloads.generate import bf16_bits_to_f32, f32_to_bf16_bits
    wl = dataclasses.replace(get_workload("tiny"), grid_h=1, grid_w=1024, chunk_frames=4, capacity_frames=8,
                             head_dim=128, n_kv_heads=6, n_q_heads=12)
    gpu, ora = _caches(rtv_lib, wl, max_global_frames=4 * wl.chunk_frames, prob_terms=prob_terms)
    n = wl.chunk_tokens
    rows = np.unique(np.concatenate([[0, 31, 32, 255, 256, n - 1], np.random.default_rng(9).integers(0, n, 26)]))
    for step in range(2):
        q, k, v = qkv_normal(wl, 0, step, 0)
        if step == 1:
            k = f32_to_bf16_bits(bf16_bits_to_f32(k) * np.float32(2.0)).reshape(k.shape)
        print(f"peaked prob_terms={prob_terms} step={step}", flush=True)
        gpu.append(0, to_dev_bf16(k), to_dev_bf16(v))
        ora.append(0, k, v)
        if step == 0:
            gpu.advance(0)
            ora.advance(0)
    out = gpu.attend(0, to_dev_bf16(q))
    want = ora.attend(0, q, rows=rows)
    mx, mean = attention_errors(bf16_to_np_f32(out)[rows], want)
    print(f"peaked prob_terms={prob_terms} attention max={mx:.3e} mean={mean:.3e}", flush=True)
    if prob_terms == 2:
        assert mx <= MAX_ABS and mean <= MEAN_ABS
