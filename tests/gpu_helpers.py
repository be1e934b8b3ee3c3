"""Helpers shared by the GPU tests: moving seeded inputs to the device and
reading the ring back in the oracle's (token, head, dim) order."""
from __future__ import annotations

import numpy as np
import torch


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_to_np_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def vt_key(p: np.ndarray) -> np.ndarray:
    """Key index held by byte p of a transposed V tile row (layout documented
    in include/rtv.h)."""
    h = p // 32
    b = p % 32
    return 32 * (b >> 4) + 8 * ((b >> 2) & 3) + 4 * h + (b & 3)


_POS_OF_KEY = np.empty(64, dtype=np.int64)
_POS_OF_KEY[vt_key(np.arange(64))] = np.arange(64)


def ring_rows(cache, layer: int, slots: np.ndarray):
    """Codes and scales at the given slots: (kc [n,H,D], ks [n,H], vc [n,H,D], vs [n,H])."""
    kc, vc, ks, vs = cache.ring_tensors(layer)
    slots_t = torch.as_tensor(slots, device=kc.device)
    k_codes = kc[:, slots_t, :].permute(1, 0, 2).cpu().numpy()
    k_scales = ks[:, slots_t].permute(1, 0).cpu().numpy()
    v_scales = vs[:, slots_t].permute(1, 0).cpu().numpy()
    vt = vc.cpu().numpy().transpose(0, 1, 3, 2)          # [H, tiles, 64 positions, D]
    v_codes = vt[:, slots // 64, _POS_OF_KEY[slots % 64], :].transpose(1, 0, 2)
    return k_codes, k_scales, v_codes, v_scales


def attention_errors(got: np.ndarray, want: np.ndarray):
    err = np.abs(got.astype(np.float64) - want)
    return float(err.max()), float(err.mean())
