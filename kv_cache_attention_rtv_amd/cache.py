"""RtvCache: a torch-facing handle over the C ABI (argument marshalling only).

torch supplies the device memory (the cache arena is a torch uint8 tensor, so
the allocation is visible to torch's allocator) and the stream; every step of
the path runs in the library's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import abi


@dataclass(frozen=True)
class RtvConfig:
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    tokens_per_frame: int
    chunk_frames: int
    capacity_frames: int
    max_global_frames: int
    rope_base: float = 10000.0
    query_terms: int = 1        # 2: two-term e4m3 queries on every window
    prob_terms: int = 0         # 0: one-code weights checked for peaked rows (recomputed with two
                                # terms); 1: one code, unchecked; 2: two terms on every window
    # optional float32 [max_global_frames * T, D/2, 2] (cos, sin) table; None: the library's own
    rope_table: object = None

    def to_c(self) -> abi.rtv_config:
        table = None
        if self.rope_table is not None:
            import numpy as np

            table = np.ascontiguousarray(self.rope_table, dtype=np.float32)
            want = (self.max_global_frames * self.tokens_per_frame, self.head_dim // 2, 2)
            if table.shape != want:
                raise ValueError(f"rope_table must be {want}, got {table.shape}")
        c = abi.rtv_config(self.n_layers, self.n_q_heads, self.n_kv_heads, self.head_dim,
                           self.tokens_per_frame, self.chunk_frames, self.capacity_frames,
                           self.max_global_frames, int(self.query_terms), int(self.prob_terms),
                           float(self.rope_base), table.ctypes.data if table is not None else None)
        c._table = table           # kept alive with the struct until the cache is created
        return c

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.tokens_per_frame


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _tok_stride(t: torch.Tensor, heads: int, head_dim: int, what: str) -> int:
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{what} must be a bf16 CUDA tensor")
    if t.dim() != 3 or t.shape[1] != heads or t.shape[2] != head_dim:
        raise ValueError(f"{what} must be [n_tokens, {heads}, {head_dim}], got {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != head_dim:
        raise ValueError(f"{what}: heads and dims must be packed (token stride may be larger)")
    return int(t.stride(0))


class RtvCache:
    def __init__(self, cfg: RtvConfig, device=None, stream=None):
        self.cfg = cfg
        self._c = cfg.to_c()
        self.device = torch.device(device if device is not None else "cuda")
        nbytes = abi.rtv_cache_bytes(self._c)
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.handle = abi.rtv_cache_create(self._c, self.arena.data_ptr(), nbytes, _stream(stream))

    def close(self):
        if getattr(self, "handle", None):
            abi.rtv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- hot path ----------------------------------------------------------
    def append(self, layer: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        c = self.cfg
        ks = _tok_stride(k, c.n_kv_heads, c.head_dim, "k")
        vs = _tok_stride(v, c.n_kv_heads, c.head_dim, "v")
        abi.rtv_append_rope_quant(self.handle, layer, k.data_ptr(), ks, v.data_ptr(), vs,
                                  k.shape[0], _stream(stream))

    def attend(self, layer: int, q: torch.Tensor, out: torch.Tensor | None = None,
               max_window_frames: int = 0, stream=None) -> torch.Tensor:
        c = self.cfg
        qs = _tok_stride(q, c.n_q_heads, c.head_dim, "q")
        if out is None:
            out = torch.empty_like(q, memory_format=torch.contiguous_format)
        os_ = _tok_stride(out, c.n_q_heads, c.head_dim, "out")
        abi.rtv_attend(self.handle, layer, q.data_ptr(), qs, out.data_ptr(), os_,
                       max_window_frames, _stream(stream))
        return out

    def advance(self, layer: int = -1, stream=None):
        abi.rtv_advance(self.handle, layer, _stream(stream))

    # -- device-resident ring state (graph capture) -------------------------
    def device_state_begin(self, stream=None):
        """Move the ring state of every layer into device memory: append, attend
        and advance then read and move it in their kernels, so that a captured
        sequence of them replays correctly step after step.  Synchronizes."""
        abi.rtv_device_state_begin(self.handle, _stream(stream))

    def device_state_end(self, stream=None):
        """Copy the ring state back to the host and leave the device-state mode.
        Synchronizes; raises RtvError(RTV_ERR_STATE) if a call in the mode ran
        past the RoPE table (its kernels wrote nothing)."""
        abi.rtv_device_state_end(self.handle, _stream(stream))

    # -- inspection ----------------------------------------------------------
    def layout(self, layer: int) -> abi.rtv_layout:
        return abi.rtv_cache_layout(self.handle, layer)

    def window(self, layer: int, max_window_frames: int = 0) -> abi.rtv_window:
        return abi.rtv_cache_window(self.handle, layer, max_window_frames)

    def peaked_units(self, stream=None) -> int:
        """Query tiles the latest attend flagged as peaked and recomputed (synchronizes)."""
        return abi.rtv_cache_peaked_units(self.handle, _stream(stream))

    def _view(self, ptr: int, nbytes: int) -> torch.Tensor:
        off = ptr - self.arena.data_ptr()
        assert 0 <= off and off + nbytes <= self.arena.numel()
        return self.arena[off: off + nbytes]

    def ring_tensors(self, layer: int):
        """Views into the arena: (k_codes [H,Sp,D] u8, v_codes [H,Sp/64,D,64] u8,
        k_scales [H,Sp] f32, v_scales [H,Sp] f32)."""
        L = self.layout(layer)
        c = self.cfg
        H, D, Sp = c.n_kv_heads, c.head_dim, L.slots_padded
        kc = self._view(L.k_codes, H * Sp * D).view(H, Sp, D)
        vc = self._view(L.v_codes, H * Sp * D).view(H, Sp // 64, D, 64)
        ks = self._view(L.k_scales, H * Sp * 4).view(torch.float32).view(H, Sp)
        vs = self._view(L.v_scales, H * Sp * 4).view(torch.float32).view(H, Sp)
        return kc, vc, ks, vs
