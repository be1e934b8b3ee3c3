"""Seeded input generators (numpy; bf16 values are carried as uint16 bit patterns).

Every draw is keyed by ``np.random.default_rng([seed, layer, step, call, tensor])``
so that any (layer, step, call) can be regenerated on its own.  Nothing here
rotates, quantizes or attends: the arrays are raw inputs to both the oracle and
the GPU library.
"""
from __future__ import annotations

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_X, TENSOR_W, TENSOR_O, TENSOR_WO = 0, 1, 2, 3, 4, 5, 6
# keys for the per-layer choices of the stress workload
_OUTLIER_CHANNELS, _ZERO_ROWS = 101, 102


def seed_key(seed: int, layer: int, step: int, call: int, tensor: int) -> list:
    return [int(seed), int(layer), int(step), int(call), int(tensor)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(key: list, shape) -> np.ndarray:
    rng = np.random.default_rng(key)
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def query_normal(wl, layer: int, step: int, call: int, seed: int = 0) -> np.ndarray:
    """Q [chunk_tokens, n_q_heads, head_dim], N(0,1) rounded to bf16."""
    shape = (wl.chunk_tokens, wl.n_q_heads, wl.head_dim)
    return _normal_bf16(seed_key(seed, layer, step, call, TENSOR_Q), shape)


def qkv_normal(wl, layer: int, step: int, call: int, seed: int = 0):
    """(Q, K, V) for one call; K/V are [chunk_tokens, n_kv_heads, head_dim]."""
    q = query_normal(wl, layer, step, call, seed)
    shape = (wl.chunk_tokens, wl.n_kv_heads, wl.head_dim)
    if wl.kv_dist == "normal":
        k = _normal_bf16(seed_key(seed, layer, step, call, TENSOR_K), shape)
        v = _normal_bf16(seed_key(seed, layer, step, call, TENSOR_V), shape)
    elif wl.kv_dist == "student_t_outliers":
        k, v = kv_student_t_outliers(wl, layer, step, call, seed)
    else:  # pragma: no cover
        raise ValueError(wl.kv_dist)
    return q, k, v


def outlier_channels(wl, layer: int, seed: int = 0) -> np.ndarray:
    """Four outlier channels per KV head, chosen once per layer: [n_kv_heads, 4]."""
    rng = np.random.default_rng([seed, layer, _OUTLIER_CHANNELS])
    return np.stack([rng.choice(wl.head_dim, size=4, replace=False)
                     for _ in range(wl.n_kv_heads)])


def kv_student_t_outliers(wl, layer: int, step: int, call: int, seed: int = 0):
    """K/V drawn Student-t (nu = 3), 4 channels per head scaled x20, 1 % of the
    token rows set to +0 in both K and V (all heads)."""
    shape = (wl.chunk_tokens, wl.n_kv_heads, wl.head_dim)
    chans = outlier_channels(wl, layer, seed)
    out = []
    for tensor in (TENSOR_K, TENSOR_V):
        rng = np.random.default_rng(seed_key(seed, layer, step, call, tensor))
        x = rng.standard_t(3, size=shape).astype(np.float32)
        for h in range(wl.n_kv_heads):
            x[:, h, chans[h]] *= np.float32(20.0)
        out.append(x)
    rng = np.random.default_rng(seed_key(seed, layer, step, call, _ZERO_ROWS))
    n_zero = max(1, wl.chunk_tokens // 100)
    rows = rng.choice(wl.chunk_tokens, size=n_zero, replace=False)
    for x in out:
        x[rows] = 0.0
    return f32_to_bf16_bits(out[0]), f32_to_bf16_bits(out[1])


def zero_rows(wl, layer: int, step: int, call: int, seed: int = 0) -> np.ndarray:
    """Token rows that kv_student_t_outliers zeroes for this call."""
    rng = np.random.default_rng(seed_key(seed, layer, step, call, _ZERO_ROWS))
    n_zero = max(1, wl.chunk_tokens // 100)
    return np.sort(rng.choice(wl.chunk_tokens, size=n_zero, replace=False))


def projection_inputs(wl, layer: int = 0, step: int = 0, seed: int = 0):
    """X [chunk_tokens, hidden] ~ N(0,1) and W [hidden, proj_width] ~ N(0, 1/hidden),
    both rounded to bf16."""
    rng = np.random.default_rng(seed_key(seed, layer, step, 0, TENSOR_X))
    x = f32_to_bf16_bits(rng.standard_normal((wl.chunk_tokens, wl.hidden), dtype=np.float32))
    rng = np.random.default_rng(seed_key(seed, layer, 0, 0, TENSOR_W))
    w = rng.standard_normal((wl.hidden, wl.proj_width), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(wl.hidden))
    return x, f32_to_bf16_bits(w)


def out_projection_inputs(n_tokens: int, in_cols: int, hidden: int, layer: int = 0, step: int = 0, seed: int = 0):
    """One GPU's share of the out-projection: O [n_tokens, in_cols] ~ N(0,1) (the
    attention output of its query heads) and Wo [in_cols, hidden] ~ N(0, 1/in_cols),
    both rounded to bf16."""
    rng = np.random.default_rng(seed_key(seed, layer, step, 0, TENSOR_O))
    o = f32_to_bf16_bits(rng.standard_normal((n_tokens, in_cols), dtype=np.float32))
    rng = np.random.default_rng(seed_key(seed, layer, 0, 0, TENSOR_WO))
    w = rng.standard_normal((in_cols, hidden), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(in_cols))
    return o, f32_to_bf16_bits(w)


def device_normal_bf16(shape, seed_tuple, device):
    """N(0,1) bf16 tensor drawn on the device by torch's generator (benchmark inputs,
    where the oracle does not see the values)."""
    import torch

    g = torch.Generator(device=device)
    h = 0
    for s in seed_tuple:
        h = (h * 1000003 + int(s) + 1) % (2**63 - 1)
    g.manual_seed(h)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
