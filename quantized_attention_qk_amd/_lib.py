"""ctypes loader for libsage_attn.so (the C ABI of include/sage_attn.h).

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process, so streams and pointers agree).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before the HIP library)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsage_attn.so")

SAGE_OK = 0
SAGE_PV = {"fp16": 0, "fp8": 1, "int8": 2}
SAGE_DT = {torch.float16: 0, torch.bfloat16: 1}
SAGE_LAYOUT = {"HND": 0, "NHD": 1}

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes)
_SIGNATURES = {
    "sage_status_str": (ctypes.c_char_p, [_c_int]),
    "sage_attn_get_tiling": (_c_int, [_c_int, _c_int, _c_int] + [ctypes.POINTER(_c_int)] * 4),
    "sage_attn_workspace_bytes": (_c_size, [_c_int] * 5),
    "sage_attn_fwd": (_c_int, [_vp] * 4 + [_c_int] * 7 + [_vp, _c_size, _vp]),
    "sage_attn_fwd_f32out": (_c_int, [_vp] * 4 + [_c_int] * 7 + [_vp, _c_size, _vp]),
    "sage_smooth_quant_qk_scratch_bytes": (_c_size, [_c_int] * 4),
    "sage_attn_fwd_ex": (_c_int, [_vp] * 4 + [_c_int] * 8 + [_vp, _vp, _c_int, _vp, _c_size, _vp]),
    "sage_smooth_quant_qk": (_c_int, [_vp, _vp] + [_c_int] * 5 + [_vp] * 6 + [_c_size, _vp]),
    "sage_smooth_quant_qk_ex": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp] + [_c_int] * 4 +
                                [_vp] * 6 + [_c_size, _vp]),
    "sage_quant_v_ex": (_c_int, [_vp] + [_c_int] * 7 + [_vp, _vp, _vp, _c_size, _vp]),
    "sage_quant_v_bytes": (_c_size, [_c_int] * 5),
    "sage_quant_v_scratch_bytes": (_c_size, [_c_int] * 5),
    "sage_quant_v": (_c_int, [_vp] + [_c_int] * 6 + [_vp, _vp, _vp, _c_size, _vp]),
    "sage_attn_fwd_quantized": (_c_int, [_vp] * 7 + [_c_int] * 7 + [_vp]),
    "sage_attn_ref_rows_f32": (_c_int, [_vp] * 3 + [_c_int] * 6 + [_vp, _c_int, _vp, _vp]),
    "sage_attn_debug_s_i32": (_c_int, [_vp, _vp] + [_c_int] * 10 + [_vp, _vp]),
    "sage_attn_sq_workspace_bytes": (_c_size, [_c_int] * 5),
    "sage_attn_fwd_sq": (_c_int, [_vp] * 4 + [_c_int] * 9 + [_vp, _c_size, _vp]),
    "sage_smooth_q": (_c_int, [_vp, _vp] + [_c_int] * 6 + [_vp] * 5 + [_vp]),
    "sage_attn_fwd_quantized_sq": (_c_int, [_vp] * 8 + [_c_int] * 7 + [_vp]),
    "sage_attn_debug_s_fwd": (_c_int, [_vp, _c_size] + [_c_int] * 13 + [_vp, _vp, _vp]),
    "sage_attn_debug_fwd_f32": (_c_int, [_vp] * 4 + [_c_int] * 7 + [_vp, _c_size, _vp]),
    "sage_attn_fwd_noalloc": (_c_int, [_vp] * 4 + [_c_int] * 7 + [_vp]),
    "sage_attn_prepare": (_c_int, [_vp] * 3 + [_c_int] * 6 + [_vp, _c_size, _vp]),
    "sage_attn_attend": (_c_int, [_vp, _c_size, _vp] + [_c_int] * 7 + [_vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m quantized_attention_qk_amd.build` (needs hipcc)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGNATURES)


def status_str(code: int) -> str:
    return lib().sage_status_str(code).decode()


def check(code: int, what: str) -> None:
    if code != SAGE_OK:
        raise RuntimeError(f"{what} failed: {status_str(code)}")
