"""Pins of the oracle's ring-free cache (CPU only).

The oracle keeps a concatenated history; these tests run an independent
token-level ring of C frames next to it (a dict from slot to (frame, token))
and check that, across many wrap-arounds and window lengths, the ring's valid
slots hold exactly the oracle's window, at the slots the oracle predicts.
"""
import numpy as np
import pytest

from oracle import attention, bf16, quant, rope
from oracle.cache import OracleKVCache
from workloads import get_workload, qkv_normal


class TokenRing:
    """Independent model of a ring of C frames: writes tokens to slots and
    remembers, per slot, which (global frame, token) it holds."""

    def __init__(self, T, F, C):
        self.T, self.F, self.C = T, F, C
        self.slot = {}
        self.frame = 0      # first frame of the chunk being written
        self.valid = 0      # frames written and committed

    def write_chunk(self):
        for f in range(self.frame, self.frame + self.F):
            for t in range(self.T):
                self.slot[(f % self.C) * self.T + t] = (f, t)

    def window(self, max_frames=0):
        w = min(self.valid + self.F, self.C)
        if max_frames:
            w = min(w, max_frames)
        first = self.frame + self.F - w
        return {s: ft for s, ft in self.slot.items() if ft[0] >= first}

    def advance(self):
        self.frame += self.F
        self.valid = min(self.valid + self.F, self.C)


def _small_cache(T=6, F=2, C=6, H=1, D=4):
    return OracleKVCache(1, H, D, T, F, C, 10000.0)


def _rand_chunk(rng, n, H, D):
    from workloads import f32_to_bf16_bits
    return (f32_to_bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32)),
            f32_to_bf16_bits(rng.standard_normal((n, H, D)).astype(np.float32)))


@pytest.mark.parametrize("T,F,C", [(6, 2, 6), (5, 1, 3), (96, 4, 8), (3, 4, 12)])
def test_ring_equivalence_over_wraps(T, F, C):
    rng = np.random.default_rng(0)
    cache = OracleKVCache(1, 1, 4, T, F, C, 10000.0)
    ring = TokenRing(T, F, C)
    for step in range(3 * C // F + 3):
        k, v = _rand_chunk(rng, F * T, 1, 4)
        cache.append(0, k, v)
        ring.write_chunk()
        for maxw in sorted({0, F, C} | set(range(F, C + 1, F))):
            frames, tok, *_ = cache.window(0, maxw)
            slots = cache.expected_slots(0, maxw)
            want = ring.window(maxw)
            assert len(slots) == len(set(slots.tolist())) == len(want)
            for s, f, t in zip(slots.tolist(), frames.tolist(), tok.tolist()):
                assert want[s] == (f, t)
        cache.advance(0)
        ring.advance()


def test_window_growth_and_repeated_append():
    wl = get_workload("tiny")
    cache = OracleKVCache(1, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame,
                          wl.chunk_frames, wl.capacity_frames, wl.rope_base)
    sizes = []
    for step in range(4):
        _, k, v = qkv_normal(wl, 0, step, 0)
        cache.append(0, k, v)
        first = cache.current[0].k_codes.copy()
        _, k2, v2 = qkv_normal(wl, 0, step, 1)
        cache.append(0, k2, v2)     # a second call of the same step replaces the chunk
        assert not np.array_equal(first, cache.current[0].k_codes)
        sizes.append(cache.window_frames(0))
        cache.advance(0)
    assert sizes == [4, 8, 8, 8]
    assert len(cache.hist[0]) == 4


def test_append_is_rope_then_quantize_at_chunk_positions():
    wl = get_workload("tiny")
    cache = OracleKVCache(1, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame,
                          wl.chunk_frames, wl.capacity_frames, wl.rope_base)
    for step in range(3):
        _, k, v = qkv_normal(wl, 0, step, 0)
        e = cache.append(0, k, v)
        pos = np.arange(step * wl.chunk_tokens, (step + 1) * wl.chunk_tokens)
        c, s = rope.cos_sin_table(pos, wl.head_dim, wl.rope_base)
        kc, ks = quant.quantize_rows(rope.apply_rope(bf16.to_f32(k), c, s))
        vc, vs = quant.quantize_rows(bf16.to_f32(v))
        assert np.array_equal(kc, e.k_codes) and np.array_equal(ks, e.k_scales)
        assert np.array_equal(vc, e.v_codes) and np.array_equal(vs, e.v_scales)
        cache.advance(0)


def test_attend_equals_attention_over_assembled_window():
    wl = get_workload("tiny")
    cache = OracleKVCache(1, wl.n_kv_heads, wl.head_dim, wl.tokens_per_frame,
                          wl.chunk_frames, wl.capacity_frames, wl.rope_base)
    kept = []
    for step in range(4):
        q, k, v = qkv_normal(wl, 0, step, 0)
        e = cache.append(0, k, v)
        kept.append(e)
        rows = [0, 17, 383]
        got = cache.attend(0, q, rows=rows)
        # assemble the window by hand: last min(4*(step+1), 8) frames = last chunks
        chunks = kept[-2:] if step >= 1 else kept[-1:]
        kd = np.concatenate([quant.dequantize_rows(c.k_codes, c.k_scales) for c in chunks])
        vd = np.concatenate([quant.dequantize_rows(c.v_codes, c.v_scales) for c in chunks])
        pos = np.arange(step * 384, step * 384 + 384)
        c_, s_ = rope.cos_sin_table(pos, wl.head_dim, wl.rope_base)
        qr = rope.apply_rope(bf16.to_f32(q), c_, s_)
        want = attention.attend(qr, kd, vd, rows=rows)
        assert np.allclose(got, want, rtol=0, atol=1e-12)
        cache.advance(0)


def test_relative_positions_survive_the_cache():
    """Scores between a query and a cached key depend only on their distance:
    shifting the whole stream by whole chunks leaves q.k unchanged up to the
    float32 rounding of RoPE and the e4m3 code of K."""
    T, F, C, D = 4, 2, 4, 8
    rng = np.random.default_rng(9)
    k, v = _rand_chunk(rng, F * T, 1, D)
    q, _ = _rand_chunk(rng, F * T, 1, D)
    results = []
    for lead in (0, 3):
        cache = OracleKVCache(1, 1, D, T, F, C, 10000.0)
        for _ in range(lead):
            cache.append(0, *_rand_chunk(rng, F * T, 1, D))
            cache.advance(0)
        cache.append(0, k, v)
        qr = cache.rotated_queries(0, q)
        _, _, kc, ks, _, _ = cache.window(0, F)
        kd = quant.dequantize_rows(kc[:, 0, :], ks[:, 0])
        results.append(qr[:, 0, :].astype(np.float64) @ kd.T)
    assert np.allclose(results[0], results[1], atol=0.25 * np.abs(results[0]).max())
    assert np.corrcoef(results[0].ravel(), results[1].ravel())[0, 1] > 0.99
