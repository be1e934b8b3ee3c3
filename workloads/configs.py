"""Shapes of the five synthetic workloads.

The serving system these shapes stand in for produces 704x1088 video as
four-frame chunks, one chunk per diffusion step, with 240 attention calls per
step (page "Runway: Πώς ένα AI 57 δισ. παραμέτρων παράγει βίντεο στα 24 fps",
sections "Τέσσερα νέα καρέ κάθε 166,7 χιλιοστά του δευτερολέπτου" and
"Από οκτώ H100 σε τέσσερις").  The pages state no head count, head size,
latent grid or cache capacity; those below are synthetic choices:
a 44x68 latent grid per frame, 12 KV heads of size 128 per GPU (a 48-head
layer split four ways), a 16-frame ring.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    chunk_frames: int
    capacity_frames: int
    rope_base: float = 10000.0
    # how K/V values are drawn: "normal" (N(0,1)) or "student_t_outliers"
    kv_dist: str = "normal"
    # calls of (append, attend) per layer per step, then one advance per layer
    calls_per_layer: int = 1
    # number of chunks streamed (steps) in the reference run of this workload
    steps: int = 1
    # projection workload only: hidden size and projection width
    hidden: int = 0
    proj_width: int = 0
    # window-length schedule in frames (0 = all valid frames)
    window_cycle: tuple = field(default_factory=tuple)

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def chunk_tokens(self) -> int:
        return self.chunk_frames * self.tokens_per_frame

    @property
    def capacity_tokens(self) -> int:
        return self.capacity_frames * self.tokens_per_frame

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    "tiny": Workload(
        name="tiny",
        description="1 layer, 2 heads x 64, 8x12 grid (96 tokens/frame), "
        "4-frame chunks (384 tokens), ring of 8 frames, 12 chunks so the ring wraps",
        n_layers=1, n_q_heads=2, n_kv_heads=2, head_dim=64,
        grid_h=8, grid_w=12, chunk_frames=4, capacity_frames=8, steps=12,
    ),
    "layer": Workload(
        name="layer",
        description="1 layer at one GPU's head share: 12 heads x 128, 44x68 grid "
        "(2992 tokens/frame), 11968-token chunk, ring of 16 frames (47872 slots), full ring",
        n_layers=1, n_q_heads=12, n_kv_heads=12, head_dim=128,
        grid_h=44, grid_w=68, chunk_frames=4, capacity_frames=16, steps=4,
    ),
    "step": Workload(
        name="step",
        description="full step: the layer shape over 60 layers x 4 (append, attend) "
        "calls = 240 calls per step, ring valid length 0 -> full over the first 4 steps",
        n_layers=60, n_q_heads=12, n_kv_heads=12, head_dim=128,
        grid_h=44, grid_w=68, chunk_frames=4, capacity_frames=16,
        calls_per_layer=4, steps=50,
    ),
    "stress": Workload(
        name="stress",
        description="FP8 stress: layer shape, K/V Student-t (nu=3) with 4 x20 outlier "
        "channels per head and 1% all-zero tokens, ring of 24 frames, window cycling 4..24",
        n_layers=1, n_q_heads=12, n_kv_heads=12, head_dim=128,
        grid_h=44, grid_w=68, chunk_frames=4, capacity_frames=24,
        kv_dist="student_t_outliers", steps=12,
        window_cycle=(4, 8, 12, 16, 20, 24),
    ),
    "proj": Workload(
        name="proj",
        description="projection + cache: X [11968 x 6144] bf16 -> per-tensor e4m3, "
        "FP8 GEMM with W_qkv [6144 x 4608] e4m3, append of its K/V columns, "
        "attention of 24 query heads over 12 KV heads (GQA 2:1), ring of 32 frames",
        n_layers=1, n_q_heads=24, n_kv_heads=12, head_dim=128,
        grid_h=44, grid_w=68, chunk_frames=4, capacity_frames=32, steps=8,
        hidden=6144, proj_width=4608,
    ),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError as exc:  # pragma: no cover - message only
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from exc
