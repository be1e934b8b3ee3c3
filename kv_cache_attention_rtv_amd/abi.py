"""ctypes binding of librtv.so: the C ABI of include/rtv.h under the same names.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  The library must have been built (``python
kv_cache_attention_rtv_amd/build.py``); importing this module fails loudly if it
is missing, and there is no fallback implementation.
"""
from __future__ import annotations

import ctypes

# torch's HIP runtime is loaded before the library, so the library binds to
# the runtime that owns the tensors it is handed (a second runtime loaded
# first would see torch's device pointers as invalid)
import torch  # noqa: F401
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# RTV_LIB may name another build of the same library (e.g. a profiling build)
LIB_PATH = os.environ.get("RTV_LIB") or os.path.join(_HERE, "librtv.so")

RTV_OK = 0
RTV_ERR_INVALID_ARG = -1
RTV_ERR_BUFFER = -2
RTV_ERR_HIP = -3
RTV_ERR_STATE = -4
RTV_ERR_UNSUPPORTED = -5


class RtvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_string(status)})")


class rtv_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("tokens_per_frame", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32),
        ("capacity_frames", ctypes.c_int32),
        ("max_global_frames", ctypes.c_int32),
        ("query_terms", ctypes.c_int32),
        ("prob_terms", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("rope_cos_sin_host", ctypes.c_void_p),
    ]


class rtv_layout(ctypes.Structure):
    _fields_ = [
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("slots", ctypes.c_int64),
        ("slots_padded", ctypes.c_int64),
        ("next_global_frame", ctypes.c_int64),
        ("head_frame", ctypes.c_int32),
        ("committed_frames", ctypes.c_int32),
        ("appended", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class rtv_window(ctypes.Structure):
    _fields_ = [
        ("window_frames", ctypes.c_int32),
        ("n_segments", ctypes.c_int32),
        ("seg_start", ctypes.c_int64 * 2),
        ("seg_len", ctypes.c_int64 * 2),
        ("write_slot", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python kv_cache_attention_rtv_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "rtv_cache_bytes": (I32, [ctypes.POINTER(rtv_config), ctypes.POINTER(SZ)]),
        "rtv_cache_create": (I32, [ctypes.POINTER(rtv_config), P, SZ, P, ctypes.POINTER(P)]),
        "rtv_destroy": (I32, [P]),
        "rtv_append_rope_quant": (I32, [P, I32, P, I64, P, I64, I32, P]),
        "rtv_attend": (I32, [P, I32, P, I64, P, I64, I32, P]),
        "rtv_advance": (I32, [P, I32, P]),
        "rtv_device_state_begin": (I32, [P, P]),
        "rtv_device_state_end": (I32, [P, P]),
        "rtv_cache_layout": (I32, [P, I32, ctypes.POINTER(rtv_layout)]),
        "rtv_cache_window": (I32, [P, I32, I32, ctypes.POINTER(rtv_window)]),
        "rtv_cache_peaked_units": (I32, [P, ctypes.POINTER(I32), P]),
        "rtv_ring_window": (I32, [I64, I32, I32, I32, I32, I32, ctypes.POINTER(rtv_window)]),
        "rtv_rope_fill_host": (I32, [I32, ctypes.c_double, I64, I64, P]),
        "rtv_encode_e4m3": (I32, [P, P, I64, P]),
        "rtv_status_string": (ctypes.c_char_p, [I32]),
        "rtv_quant_workspace_bytes": (SZ, [I64]),
        "rtv_quant_fp8_per_tensor": (I32, [P, I64, P, P, P, P]),
        "rtv_quant_fp8_per_tensor_static": (I32, [P, I64, P, P, P]),
        "rtv_gemm_fp8": (I32, [P, P, P, P, P, I32, I32, I32, I64, P]),
        "rtv_qkv_gemm_append": (I32, [P, I32, P, P, P, P, I32, I32, I32, P, I64, P]),
    }
    missing = []
    for name, (res, args) in sigs.items():
        try:
            fn = getattr(lib, name)
        except AttributeError:
            missing.append(name)
            continue
        fn.restype = res
        fn.argtypes = args
    lib.rtv_missing_symbols = tuple(missing)
    return lib


lib = _load()
EXPORTED = (
    "rtv_cache_bytes", "rtv_cache_create", "rtv_destroy", "rtv_append_rope_quant",
    "rtv_attend", "rtv_advance", "rtv_device_state_begin", "rtv_device_state_end", "rtv_cache_layout",
    "rtv_cache_window", "rtv_cache_peaked_units", "rtv_ring_window",
    "rtv_rope_fill_host", "rtv_encode_e4m3", "rtv_status_string",
    "rtv_quant_workspace_bytes", "rtv_quant_fp8_per_tensor", "rtv_quant_fp8_per_tensor_static", "rtv_gemm_fp8",
    "rtv_qkv_gemm_append",
)


def status_string(status: int) -> str:
    return lib.rtv_status_string(int(status)).decode()


def check(status: int, what: str) -> None:
    if status != RTV_OK:
        raise RtvError(status, what)


# ---- same-name wrappers (status codes are raised as RtvError) ---------------
def rtv_cache_bytes(cfg: rtv_config) -> int:
    out = ctypes.c_size_t()
    check(lib.rtv_cache_bytes(ctypes.byref(cfg), ctypes.byref(out)), "rtv_cache_bytes")
    return out.value


def rtv_cache_create(cfg: rtv_config, dev_buf: int, nbytes: int, stream: int) -> int:
    h = ctypes.c_void_p()
    check(lib.rtv_cache_create(ctypes.byref(cfg), dev_buf, nbytes, stream, ctypes.byref(h)),
          "rtv_cache_create")
    return h.value


def rtv_destroy(handle: int) -> None:
    check(lib.rtv_destroy(handle), "rtv_destroy")


def rtv_append_rope_quant(handle, layer, k_ptr, k_stride, v_ptr, v_stride, n_tokens, stream):
    check(lib.rtv_append_rope_quant(handle, layer, k_ptr, k_stride, v_ptr, v_stride, n_tokens, stream),
          "rtv_append_rope_quant")


def rtv_attend(handle, layer, q_ptr, q_stride, out_ptr, out_stride, max_window_frames, stream):
    check(lib.rtv_attend(handle, layer, q_ptr, q_stride, out_ptr, out_stride, max_window_frames, stream),
          "rtv_attend")


def rtv_advance(handle, layer, stream):
    check(lib.rtv_advance(handle, layer, stream), "rtv_advance")


def rtv_device_state_begin(handle, stream):
    check(lib.rtv_device_state_begin(handle, stream), "rtv_device_state_begin")


def rtv_device_state_end(handle, stream):
    check(lib.rtv_device_state_end(handle, stream), "rtv_device_state_end")


def rtv_cache_layout(handle, layer) -> rtv_layout:
    out = rtv_layout()
    check(lib.rtv_cache_layout(handle, layer, ctypes.byref(out)), "rtv_cache_layout")
    return out


def rtv_cache_window(handle, layer, max_window_frames=0) -> rtv_window:
    out = rtv_window()
    check(lib.rtv_cache_window(handle, layer, max_window_frames, ctypes.byref(out)), "rtv_cache_window")
    return out


def rtv_cache_peaked_units(handle, stream) -> int:
    out = ctypes.c_int32()
    check(lib.rtv_cache_peaked_units(handle, ctypes.byref(out), stream), "rtv_cache_peaked_units")
    return out.value


def rtv_ring_window(next_global_frame, committed, tokens_per_frame, chunk_frames, capacity_frames,
                    max_window_frames=0) -> rtv_window:
    out = rtv_window()
    check(lib.rtv_ring_window(next_global_frame, committed, tokens_per_frame, chunk_frames,
                              capacity_frames, max_window_frames, ctypes.byref(out)),
          "rtv_ring_window")
    return out


def rtv_rope_fill_host(head_dim, rope_base, pos0, npos):
    import numpy as np

    out = np.empty((npos, head_dim // 2, 2), dtype=np.float32)
    check(lib.rtv_rope_fill_host(head_dim, rope_base, pos0, npos, out.ctypes.data), "rtv_rope_fill_host")
    return out


def rtv_encode_e4m3(x_ptr, codes_ptr, n, stream):
    check(lib.rtv_encode_e4m3(x_ptr, codes_ptr, n, stream), "rtv_encode_e4m3")


def rtv_quant_workspace_bytes(n) -> int:
    return int(lib.rtv_quant_workspace_bytes(n))


def rtv_quant_fp8_per_tensor(x_ptr, n, codes_ptr, scale_ptr, ws_ptr, stream):
    check(lib.rtv_quant_fp8_per_tensor(x_ptr, n, codes_ptr, scale_ptr, ws_ptr, stream),
          "rtv_quant_fp8_per_tensor")


def rtv_quant_fp8_per_tensor_static(x_ptr, n, codes_ptr, scale_ptr, stream):
    check(lib.rtv_quant_fp8_per_tensor_static(x_ptr, n, codes_ptr, scale_ptr, stream),
          "rtv_quant_fp8_per_tensor_static")


def rtv_gemm_fp8(a_ptr, sa_ptr, bt_ptr, sb_ptr, c_ptr, M, N, K, ldc, stream):
    check(lib.rtv_gemm_fp8(a_ptr, sa_ptr, bt_ptr, sb_ptr, c_ptr, M, N, K, ldc, stream), "rtv_gemm_fp8")


def rtv_qkv_gemm_append(handle, layer, x_ptr, sx_ptr, wt_ptr, sw_ptr, n_tokens, k_dim, q_cols,
                        q_ptr, q_tok_stride, stream):
    check(lib.rtv_qkv_gemm_append(handle, layer, x_ptr, sx_ptr, wt_ptr, sw_ptr, n_tokens, k_dim, q_cols,
                                  q_ptr, q_tok_stride, stream), "rtv_qkv_gemm_append")
