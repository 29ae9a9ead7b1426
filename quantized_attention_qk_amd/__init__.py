"""MI355X (gfx950) SageAttention forward pass: smoothed per-block INT8 Q K^T,
online softmax, FP16, FP8 E4M3 or INT8 P~V, optionally with Q smoothed per
block too, behind a C ABI (include/sage_attn.h).

Importing this package does not require a GPU; calling into it does, and it
fails loudly (RuntimeError) when the HIP library is missing or no device is
visible.  There is no CPU fallback.
"""
from .api import (attend, debug_s_fwd, debug_s_i32, prepare, quant_v, ref_rows, sage_attn,  # noqa: F401
                  sage_attn_quantized, smooth_q, smooth_quant_qk, tiling, untile_v,
                  workspace_bytes)
from .adaptive import choose_mode, load_modes, save_modes, select_pv_modes  # noqa: F401
