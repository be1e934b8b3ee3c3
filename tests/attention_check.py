"""The attention tolerance of the contract, and relative bounds that give it teeth.

Contract: max |err| <= 2e-2 and mean |err| <= 2e-3 against float64 attention on
the dequantized cache.  On long N(0,1) windows the outputs themselves are small
(RMS about 8e-3 over 47872 keys), so an output scaled by 0.7 would still pass
those absolute bounds.  Every attention check therefore also holds the error to
a fraction of the output's own size over the checked rows:
    mean |err| <= 0.1 * mean |O|   and   max |err| <= 0.25 * max |O|.
Workloads with heavy-tailed V are checked with the errors divided by the
window's max |V| (`normalise`) against the same absolute bounds.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_MEAN = 0.1
REL_MAX = 0.25


def attention_report(got, want, normalise=None) -> dict:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    scale = 1.0 if normalise is None else float(normalise)
    return {
        "max": float(err.max()) / scale,
        "mean": float(err.mean()) / scale,
        "rel_mean": float(err.mean() / max(np.abs(want).mean(), 1e-30)),
        "rel_max": float(err.max() / max(np.abs(want).max(), 1e-30)),
    }


def attention_ok(r: dict) -> bool:
    return (r["max"] <= MAX_ABS and r["mean"] <= MEAN_ABS and r["rel_mean"] <= REL_MEAN
            and r["rel_max"] <= REL_MAX)


def check_attention(got, want, label: str = "", normalise=None) -> dict:
    """Assert the contract's bounds and the relative bounds; returns the figures."""
    r = attention_report(got, want, normalise)
    print(f"{label} attention max={r['max']:.3e} mean={r['mean']:.3e} "
          f"rel_mean={r['rel_mean']:.3e} rel_max={r['rel_max']:.3e}", flush=True)
    assert attention_ok(r), (label, r)
    return r
