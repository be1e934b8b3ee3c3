"""torch-facing wrappers of the projection entry points (argument marshalling
only): per-tensor e4m3 quantization and the FP8 GEMM, both run by the library's
kernels on the given stream."""
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
