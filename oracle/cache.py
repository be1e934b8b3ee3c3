"""Ring-free KV cache: an explicitly concatenated history of committed chunks.

What the pages describe (page "Runway explains how it serves a 57B video model
in real time", fourth paragraph; page "Runway: Πώς ένα AI 57 δισ. παραμέτρων
παράγει βίντεο στα 24 fps", section "Από οκτώ H100 σε τέσσερις"): the cache
receives each new four-frame chunk's K/V once, with RoPE and FP8 quantization
applied at that moment, and keeps a bounded window of recent frames by moving a
head index in a circular buffer instead of copying.  This oracle reaches the
same window without any buffer arithmetic:

* ``append`` rotates K, quantizes K and V, and stores them as the layer's
  *current* chunk (a second append before ``advance`` replaces it, the way the
  repeated calls of one diffusion step overwrite the same chunk);
* ``advance`` pushes the current chunk onto the history and counts its frames
  as committed, ``committed = min(committed + F, C)``; nothing is ever popped;
* the window of an ``attend`` is the last W frames of (history + current), with
  ``W = min(committed + F, C, max_window_frames or C)``.

``expected_slots`` gives, for every window token (global frame g, token t),
the slot (g mod C) * T + t a ring of C frames would use.  It is only used to
check a ring read back from elsewhere; the oracle never stores by slot.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import attention, bf16, quant, rope


@dataclass
class ChunkEntry:
    global_frame: int
    k_codes: np.ndarray   # [n, Hkv, D] uint8
    k_scales: np.ndarray  # [n, Hkv] float32
    v_codes: np.ndarray
    v_scales: np.ndarray


class OracleKVCache:
    def __init__(self, n_layers, n_kv_heads, head_dim, tokens_per_frame,
                 chunk_frames, capacity_frames, rope_base=10000.0, rope_table=None):
        """rope_table: optional float32 [positions, D/2, 2] (cos, sin) table to
        use instead of evaluating rope.cos_sin_table, so that a test can hand
        one table to both implementations."""
        if capacity_frames % chunk_frames:
            raise ValueError("capacity_frames must be a multiple of chunk_frames")
        self.n_layers = n_layers
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.T = tokens_per_frame
        self.F = chunk_frames
        self.C = capacity_frames
        self.base = rope_base
        self.hist = [[] for _ in range(n_layers)]
        self.current = [None] * n_layers
        self.next_global_frame = [0] * n_layers
        self.committed = [0] * n_layers
        self._table_cache = {}
        self.rope_table = None if rope_table is None else np.asarray(rope_table, dtype=np.float32)

    # -- RoPE table of the chunk at a global frame ---------------------------
    def chunk_table(self, global_frame):
        key = global_frame
        if key not in self._table_cache:
            pos = rope.chunk_positions(global_frame, self.F, self.T)
            if self.rope_table is not None:
                rows = self.rope_table[pos]
                self._table_cache = {key: (rows[:, :, 0].copy(), rows[:, :, 1].copy())}
            else:
                self._table_cache = {key: rope.cos_sin_table(pos, self.head_dim, self.base)}
        return self._table_cache[key]

    # -- cache upkeep --------------------------------------------------------
    def append(self, layer, k_bits, v_bits):
        """K/V [n, Hkv, D] bf16 bit patterns; n must be one chunk."""
        n = self.F * self.T
        if k_bits.shape != (n, self.n_kv_heads, self.head_dim) or v_bits.shape != k_bits.shape:
            raise ValueError("append expects one chunk of K and V")
        g = self.next_global_frame[layer]
        cos, sin = self.chunk_table(g)
        k_rot = rope.apply_rope(bf16.to_f32(k_bits), cos, sin)
        kc, ks = quant.quantize_rows(k_rot)
        vc, vs = quant.quantize_rows(bf16.to_f32(v_bits))
        self.current[layer] = ChunkEntry(g, kc, ks, vc, vs)
        return self.current[layer]

    def advance(self, layer):
        if self.current[layer] is None:
            raise RuntimeError("advance without a chunk appended")
        self.hist[layer].append(self.current[layer])
        self.current[layer] = None
        self.next_global_frame[layer] += self.F
        self.committed[layer] = min(self.committed[layer] + self.F, self.C)

    # -- the window ----------------------------------------------------------
    def window_frames(self, layer, max_window_frames=0):
        w = min(self.committed[layer] + self.F, self.C)
        if max_window_frames:
            w = min(w, max_window_frames)
        return w

    def window(self, layer, max_window_frames=0):
        """(global_frame_of_each_token, token_in_frame, kc, ks, vc, vs) of the window."""
        cur = self.current[layer]
        if cur is None:
            raise RuntimeError("attend before append")
        w = self.window_frames(layer, max_window_frames)
        history = self.hist[layer] + [cur]
        need_chunks = -(-w // self.F)
        chunks = history[-need_chunks:]
        kc = np.concatenate([c.k_codes for c in chunks])
        ks = np.concatenate([c.k_scales for c in chunks])
        vc = np.concatenate([c.v_codes for c in chunks])
        vs = np.concatenate([c.v_scales for c in chunks])
        frames = np.concatenate([
            np.repeat(np.arange(c.global_frame, c.global_frame + self.F), self.T)
            for c in chunks])
        tok = np.tile(np.arange(self.T), self.F * len(chunks))
        keep = w * self.T
        return (frames[-keep:], tok[-keep:], kc[-keep:], ks[-keep:], vc[-keep:], vs[-keep:])

    def expected_slots(self, layer, max_window_frames=0):
        frames, tok, *_ = self.window(layer, max_window_frames)
        return (frames % self.C) * self.T + tok

    # -- attention -----------------------------------------------------------
    def rotated_queries(self, layer, q_bits):
        cur = self.current[layer]
        cos, sin = self.chunk_table(cur.global_frame)
        return rope.apply_rope(bf16.to_f32(q_bits), cos, sin)

    def attend(self, layer, q_bits, max_window_frames=0, rows=None):
        """Outputs [len(rows) or n, Hq, D] float64 for the chunk's queries."""
        q_rot = self.rotated_queries(layer, q_bits)
        _, _, kc, ks, vc, vs = self.window(layer, max_window_frames)
        hq = q_rot.shape[1]
        group = hq // self.n_kv_heads
        if rows is None:
            rows = np.arange(q_rot.shape[0])
        rows = np.asarray(rows)
        out = np.empty((len(rows), hq, self.head_dim), dtype=np.float64)
        for kvh in range(self.n_kv_heads):
            k = quant.dequantize_rows(kc[:, kvh, :], ks[:, kvh])
            v = quant.dequantize_rows(vc[:, kvh, :], vs[:, kvh])
            for h in range(kvh * group, (kvh + 1) * group):
                out[:, h, :] = attention.attend_rows(q_rot[rows, h, :], k, v)
        return out
