"""torch-facing wrappers of the projection entry points (argument marshalling
only): per-tensor e4m3 quantization, the FP8 GEMM, and the FP8 QKV GEMM fused
with the cache upkeep, all run by the library's kernels on the given stream."""
from __future__ import annotations

import torch

from . import abi
from .cache import _stream


def quant_workspace(n: int, device) -> torch.Tensor:
    return torch.empty(abi.rtv_quant_workspace_bytes(n), dtype=torch.uint8, device=device)


def quant_fp8_per_tensor(x: torch.Tensor, codes: torch.Tensor | None = None,
                         scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None):
    """(codes uint8 shaped like x, scale f32 [1]) with scale = f32(amax/448)."""
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise TypeError("x must be a contiguous bf16 CUDA tensor")
    n = x.numel()
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = quant_workspace(n, x.device)
    if codes.numel() != n or codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 tensor of x's size")
    if workspace.numel() < abi.rtv_quant_workspace_bytes(n):
        raise ValueError("workspace too small")
    abi.rtv_quant_fp8_per_tensor(x.data_ptr(), n, codes.data_ptr(), scale.data_ptr(),
                                 workspace.data_ptr(), _stream(stream))
    return codes, scale


def gemm_fp8(a: torch.Tensor, sa: torch.Tensor, bt: torch.Tensor, sb: torch.Tensor,
             out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[M][N] bf16 = sa * sb * A[M][K] @ Bt[N][K]^T (e4m3 codes, f32 accumulation)."""
    if a.dtype != torch.uint8 or bt.dtype != torch.uint8 or a.dim() != 2 or bt.dim() != 2:
        raise TypeError("a and bt must be 2-D uint8 (e4m3 code) tensors")
    if not (a.is_contiguous() and bt.is_contiguous()):
        raise ValueError("a and bt must be contiguous")
    M, K = a.shape
    N, K2 = bt.shape
    if K != K2:
        raise ValueError(f"inner sizes differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape != (M, N) or out.stride(1) != 1:
        raise ValueError("out must be a bf16 [M, N] tensor with unit column stride")
    abi.rtv_gemm_fp8(a.data_ptr(), sa.data_ptr(), bt.data_ptr(), sb.data_ptr(), out.data_ptr(),
                     M, N, K, out.stride(0), _stream(stream))
    return out


def qkv_gemm_append(cache, layer: int, x: torch.Tensor, sx: torch.Tensor, wt: torch.Tensor,
                    sw: torch.Tensor, q_cols: int, q_out: torch.Tensor | None = None, stream=None):
    """QKV = sx * sw * X[M][K] @ Wt[N][K]^T with N = q_cols + 2 * n_kv_heads * head_dim:
    the Q columns into q_out (bf16 [M, q_cols], allocated if None), the K and V
    heads through RoPE (K) and per-(token, head) e4m3 straight into the layer's
    ring as the chunk's append.  Returns q_out."""
    c = cache.cfg
    if x.dtype != torch.uint8 or wt.dtype != torch.uint8 or x.dim() != 2 or wt.dim() != 2:
        raise TypeError("x and wt must be 2-D uint8 (e4m3 code) tensors")
    if not (x.is_contiguous() and wt.is_contiguous()):
        raise ValueError("x and wt must be contiguous")
    M, K = x.shape
    N, K2 = wt.shape
    if K != K2 or N != q_cols + 2 * c.n_kv_heads * c.head_dim:
        raise ValueError(f"shapes: x {tuple(x.shape)}, wt {tuple(wt.shape)}, q_cols {q_cols}")
    if q_cols > 0 and q_out is None:
        q_out = torch.empty((M, q_cols), dtype=torch.bfloat16, device=x.device)
    q_ptr, q_stride = (q_out.data_ptr(), q_out.stride(0)) if q_cols > 0 else (0, 0)
    if q_cols > 0 and (q_out.dtype != torch.bfloat16 or q_out.shape != (M, q_cols) or q_out.stride(1) != 1):
        raise ValueError("q_out must be a bf16 [M, q_cols] tensor with unit column stride")
    abi.rtv_qkv_gemm_append(cache.handle, layer, x.data_ptr(), sx.data_ptr(), wt.data_ptr(), sw.data_ptr(),
                            M, K, q_cols, q_ptr, q_stride, _stream(stream))
    return q_out
