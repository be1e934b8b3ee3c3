"""Rotary position embedding (RoPE), rotate-half pairing, 1-D over the global
token index.

The pages say RoPE is applied once, when a frame's K/V enter the cache
(page "Runway explains how it serves a 57B video model in real time", fourth
paragraph).  They do not give the variant; the readings taken here:

* pairs are (i, i + D/2) for i < D/2 ("rotate-half");
* theta_i = base^(-2i/D), base 10000;
* the position of token t of global frame g is g*T + t (T tokens per frame);
* the rotation is counter-clockwise in the (x_i, x_{i+D/2}) plane:
      r_i       = x_i * cos - x_{i+D/2} * sin
      r_{i+D/2} = x_{i+D/2} * cos + x_i * sin
  each product and the sum/difference rounded to float32, no fused multiply-add;
* the angle pos * theta_i and its cosine and sine are evaluated in float64 by
  the C library (Python's ``math``), then rounded to float32.
"""
from __future__ import annotations

import math

import numpy as np


def inv_freq(head_dim: int, base: float) -> list:
    """theta_i = base^(-2i/D) for i < D/2, as Python floats (float64)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    return [float(base) ** (-2.0 * i / head_dim) for i in range(head_dim // 2)]


def cos_sin_f64(positions, head_dim: int, base: float):
    """float64 cos/sin of pos * theta_i, shape [len(positions), D/2] each."""
    theta = inv_freq(head_dim, base)
    positions = [int(p) for p in positions]
    c = np.empty((len(positions), len(theta)), dtype=np.float64)
    s = np.empty_like(c)
    for r, p in enumerate(positions):
        for i, th in enumerate(theta):
            ang = float(p) * th
            c[r, i] = math.cos(ang)
            s[r, i] = math.sin(ang)
    return c, s


def cos_sin_table(positions, head_dim: int, base: float):
    """float32 cos/sin table [len(positions), D/2] each (float64 values rounded once)."""
    c, s = cos_sin_f64(positions, head_dim, base)
    return c.astype(np.float32), s.astype(np.float32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate x [..., n_pos, H, D] (float32) by the per-position table [n_pos, D/2].

    ``x`` is indexed [token, head, dim]; ``cos``/``sin`` are [token, D/2].
    Returns float32; every product and sum rounded to float32.
    """
    x = np.asarray(x, dtype=np.float32)
    half = x.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float32)[:, None, :]
    s = np.asarray(sin, dtype=np.float32)[:, None, :]
    x0 = x[..., :half]
    x1 = x[..., half:]
    r = np.empty_like(x)
    a = np.multiply(x0, c, dtype=np.float32)
    b = np.multiply(x1, s, dtype=np.float32)
    r[..., :half] = np.subtract(a, b, dtype=np.float32)
    a = np.multiply(x1, c, dtype=np.float32)
    b = np.multiply(x0, s, dtype=np.float32)
    r[..., half:] = np.add(a, b, dtype=np.float32)
    return r


def chunk_positions(global_frame: int, chunk_frames: int, tokens_per_frame: int) -> np.ndarray:
    """Global token positions of the chunk that starts at ``global_frame``."""
    start = global_frame * tokens_per_frame
    return np.arange(start, start + chunk_frames * tokens_per_frame, dtype=np.int64)
