"""MI355X (gfx950) KV-cache upkeep + chunk attention.

The hot path lives in the HIP library librtv.so (C ABI: include/rtv.h); this
package binds it (``abi``, same names as the C functions) and wraps the handle
for torch callers (``RtvCache``).  Importing fails when the library has not
been built: there is no CPU fallback.
"""
from . import abi
from .abi import RtvError
from .cache import RtvCache, RtvConfig
from .projection import gemm_fp8, qkv_gemm_append, quant_fp8_per_tensor

__all__ = ["abi", "RtvError", "RtvCache", "RtvConfig", "gemm_fp8", "qkv_gemm_append", "quant_fp8_per_tensor"]
