"""CPU oracle for the SageAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
library never calls it, and it shares no code, constants or helpers with the
HIP path.
"""
from .sage_oracle import (  # noqa: F401
    Q_BLOCK, K_BLOCK, KV_TILE, MEAN_CHUNK, P_STATIC_FP8, P_STATIC_INT8,
    column_mean, quantize_int8_blocks, smooth_quant_qk, prep_v, attention, q_block_mean,
    smooth_quantize_q_blocks, q_compensation, SQ_LIMIT, SQ_FRAC_BITS,
    sage_attention, brute_attention, cos_sim, rel_l1, rmse, s_int32_tile,
    inv_sqrt_d, rope_rotate_half,
)
from .codecs import e4m3_encode, e4m3_decode, e4m3_flip_step, fp16_round, int8_flip_step  # noqa: F401
