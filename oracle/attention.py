"""Softmax attention in float64 over a dequantized key/value window.

Per query head h with KV head h // (Hq / Hkv):
    s_j = (q . k_j) / sqrt(D)
    p   = softmax(s)            (max-subtracted before exponentiation)
    o   = sum_j p_j v_j
The chunk's queries see every key of the window, the chunk itself included:
a 4-frame chunk attends to the valid cached frames and to all of its own
frames, with no mask inside the chunk (block-causal at chunk granularity).
The pages give the call count (240 attention calls per step, page
"Runway: Πώς ένα AI 57 δισ. παραμέτρων παράγει βίντεο στα 24 fps", section
"Από οκτώ H100 σε τέσσερις") but no formula; the softmax scale 1/sqrt(D) and
the absence of an intra-chunk mask are the plainest readings.
"""
from __future__ import annotations

import numpy as np


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Attention for a set of query rows of ONE head.

    q [m, D], k [L, D], v [L, D] (any float dtype; computed in float64).
    Returns o [m, D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[-1]
    s = (q @ k.T) / np.sqrt(float(d))
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows=None) -> np.ndarray:
    """Grouped-query attention.

    q [n, Hq, D], k/v [L, Hkv, D].  ``rows`` optionally selects query rows
    (indices into n); returns o [len(rows) or n, Hq, D] float64.
    """
    n, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = hq // hkv
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows)
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    for h in range(hq):
        kv = h // group
        out[:, h, :] = attend_rows(q[rows, h, :], k[:, kv, :], v[:, kv, :])
    return out
