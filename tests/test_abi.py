"""C ABI checks that need no GPU: the library loads, exports every symbol
declared in include/sage_attn.h, reports its tiling, sizes its workspace, and
rejects invalid arguments (or reports a missing device) without enqueuing.

Fake device pointers below are never dereferenced: every call returns before
any launch, either from argument validation or from the device check.
"""
import ctypes
import os
import re

import pytest
import torch

from quantized_attention_qk_amd import _lib
from quantized_attention_qk_amd._lib import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, NO_DEVICE = range(6)
P = 0x10000          # an aligned, never-dereferenced fake pointer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 10
    h = lib()
    for n in names:
        assert hasattr(h, n), n
    assert sorted(_lib.exported_symbols()) == names


def test_status_strings():
    for code, tag in [(OK, "SAGE_OK"), (INVALID, "INVALID_ARG"), (UNSUPPORTED, "UNSUPPORTED"),
                      (WORKSPACE, "WORKSPACE"), (HIP, "SAGE_ERR_HIP"), (NO_DEVICE, "NO_DEVICE")]:
        assert tag in _lib.status_str(code)
    assert "UNKNOWN" in _lib.status_str(99)


def test_tiling_contract_matches_oracle():
    import oracle
    vals = [ctypes.c_int() for _ in range(4)]
    for d in (64, 128):
        for pv in (0, 1, 2):
            assert lib().sage_attn_get_tiling(d, 0, pv, *[ctypes.byref(v) for v in vals]) == OK
            assert [v.value for v in vals] == [oracle.Q_BLOCK, oracle.K_BLOCK, oracle.KV_TILE,
                                               oracle.MEAN_CHUNK]
    assert lib().sage_attn_get_tiling(96, 0, 0, None, None, None, None) == UNSUPPORTED
    assert lib().sage_attn_get_tiling(64, 0, 7, None, None, None, None) == UNSUPPORTED


def test_workspace_sizes():
    h = lib()
    B, H, N, d = 1, 24, 16384, 128
    w16 = h.sage_attn_workspace_bytes(B, H, N, d, 0)
    w8 = h.sage_attn_workspace_bytes(B, H, N, d, 1)
    wi8 = h.sage_attn_workspace_bytes(B, H, N, d, 2)
    elems = B * H * N * d
    # Q^ + K^ (int8) + V' (fp16) at least; V^ (e4m3) is half of V'
    assert w16 >= 2 * elems + 2 * elems
    assert w8 >= 2 * elems + elems and w8 < w16
    assert wi8 == w8                      # INT8 V^ has the FP8 layout and size
    assert h.sage_attn_workspace_bytes(1, 1, 0, 64, 0) == 0
    assert h.sage_attn_workspace_bytes(1, 1, 10, 96, 0) == 0
    assert h.sage_attn_workspace_bytes(1, 1, 10, 64, 3) == 0
    assert h.sage_quant_v_bytes(1, 2, 65, 64, 0) == 2 * 2 * 64 * 128
    assert h.sage_quant_v_bytes(1, 2, 65, 64, 1) == 2 * 2 * 64 * 64
    assert h.sage_quant_v_bytes(1, 2, 65, 64, 2) == 2 * 2 * 64 * 64
    assert h.sage_quant_v_scratch_bytes(1, 2, 65, 64, 0) == 0
    assert h.sage_quant_v_scratch_bytes(1, 2, 65, 64, 2) == h.sage_quant_v_scratch_bytes(1, 2, 65, 64, 1) > 0
    assert h.sage_smooth_quant_qk_scratch_bytes(2, 3, 257, 128) == 2 * 3 * 2 * 128 * 4


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P + 0x1000, B=1, H=2, N=100, d=64, causal=0, pv=0, dtype=0,
             ws=P + 0x100000, wsb=1 << 40)
    a.update(kw)
    return lib().sage_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["N"], a["d"],
                               a["causal"], a["pv"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(ws=None), INVALID),
    (dict(q=P + 8), INVALID), (dict(o=P + 2), INVALID), (dict(ws=P + 16), INVALID),
    (dict(causal=2), INVALID), (dict(pv=3), INVALID), (dict(pv=-1), INVALID),
    (dict(dtype=5), INVALID),
    (dict(N=0), INVALID), (dict(B=0), INVALID), (dict(H=-1), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(N=(1 << 24) + 1), UNSUPPORTED),
    (dict(o=P), INVALID), (dict(wsb=1000), WORKSPACE),
])
def test_fwd_argument_validation(kw, code):
    assert fwd(**kw) == code


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_no_device_reported_after_validation():
    # valid arguments: the only failure left is the missing device
    assert fwd() == NO_DEVICE
    assert lib().sage_attn_fwd_f32out(P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 0, 0, P + 0x100000,
                                      1 << 40, None) == NO_DEVICE


def test_stage_argument_validation():
    h = lib()
    # smooth_quant_qk: scratch too small
    assert h.sage_smooth_quant_qk(P, P, 0, 1, 1, 300, 64, P, P, P, P, P, P, 16, None) == WORKSPACE
    assert h.sage_smooth_quant_qk(P, P, 0, 1, 1, 300, 64, None, P, P, P, P, P, 1 << 30, None) == INVALID
    assert h.sage_smooth_quant_qk(P, P, 0, 1, 1, 300, 96, P, P, P, P, P, P, 1 << 30, None) == UNSUPPORTED
    # quant_v: FP8 needs v_scale and scratch
    assert h.sage_quant_v(P, 0, 1, 1, 300, 64, 1, P, None, P, 1 << 30, None) == INVALID
    assert h.sage_quant_v(P, 0, 1, 1, 300, 64, 1, P, P, P, 8, None) == WORKSPACE
    assert h.sage_quant_v(P, 0, 1, 1, 300, 64, 4, P, P, P, 1 << 30, None) == INVALID
    # debug S: rectangle must be 32-aligned and inside the padded range
    assert h.sage_attn_debug_s_i32(P, P, 1, 1, 100, 64, 0, 0, 0, 32, 16, 32, P, None) == INVALID
    assert h.sage_attn_debug_s_i32(P, P, 1, 1, 100, 64, 0, 0, 96, 64, 0, 32, P, None) == INVALID
    assert h.sage_attn_debug_s_i32(P, P, 1, 1, 100, 64, 0, 1, 0, 32, 0, 32, P, None) == INVALID
    if not torch.cuda.is_available():
        assert h.sage_attn_debug_s_i32(P, P, 1, 1, 100, 64, 0, 0, 96, 32, 0, 128, P, None) == NO_DEVICE
        assert h.sage_smooth_quant_qk(P, P, 0, 1, 1, 300, 64, P, P, P, P, P, P, 1 << 30, None) == NO_DEVICE


def test_python_binding_fails_loudly_without_device():
    import quantized_attention_qk_amd as qa
    if torch.cuda.is_available():
        pytest.skip("device present")
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        qa.sage_attn(q, q, q)          # CPU tensors are rejected, never computed on the CPU


def test_untile_v_inverts_documented_layout():
    # build a tiled buffer from the documented formulas and invert it
    import numpy as np
    from quantized_attention_qk_amd import untile_v
    B, H, N, d = 1, 2, 70, 64
    nt = 2
    for mode, rowb in (("fp16", 128), ("fp8", 64)):
        nat = np.arange(B * H * nt * 64 * d).reshape(B, H, nt * 64, d)
        if mode == "fp16":
            nat = (nat % 2000).astype(np.float16)
            tiled = np.zeros((B, H, nt, d, 8, 8), np.float16)
            for t in range(nt):
                for c in range(d):
                    for kk in range(8):
                        for e in range(8):
                            key = 64 * t + 16 * (kk // 2) + 8 * (e // 4) + 4 * (kk % 2) + e % 4
                            tiled[0, :, t, c, kk ^ ((c // 2) % 8), e] = nat[0, :, key, c]
            raw = tiled.view(np.uint8).ravel()
        else:
            nat = (nat % 251).astype(np.uint8)
            tiled = np.zeros((B, H, nt, d, 64), np.uint8)
            for t in range(nt):
                for c in range(d):
                    for p in range(64):
                        key = 64 * t + 32 * ((p // 16) % 2) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
                        phys = 16 * ((p // 16) ^ ((c // 4) % 4)) + p % 16
                        tiled[0, :, t, c, phys] = nat[0, :, key, c]
            raw = tiled.ravel()
        assert raw.size == B * H * nt * d * rowb
        back = untile_v(raw, B, H, N, d, mode)
        np.testing.assert_array_equal(back, nat[:, :, :N])


def test_quantized_entry_validation():
    h = lib()
    args = [P] * 7 + [1, 2, 100, 64, 0, 0, 0, None]
    bad = list(args)
    bad[0] = None
    assert h.sage_attn_fwd_quantized(*bad) == INVALID
    bad = list(args)
    bad[13] = 3                    # out dtype
    assert h.sage_attn_fwd_quantized(*bad) == INVALID
    bad = list(args)
    bad[12] = 1                    # FP8 without v_scale
    bad[5] = None
    assert h.sage_attn_fwd_quantized(*bad) == INVALID
    bad = list(args)
    bad[10] = 80                   # d
    assert h.sage_attn_fwd_quantized(*bad) == UNSUPPORTED
    if not torch.cuda.is_available():
        assert h.sage_attn_fwd_quantized(*args) == NO_DEVICE


def test_ref_rows_validation():
    h = lib()
    args = [P, P, P, 0, 1, 2, 100, 64, 0, P, 5, P, None]
    assert h.sage_attn_ref_rows_f32(*args[:9], None, *args[10:]) == INVALID    # no rows
    bad = list(args)
    bad[3] = 2                     # dtype
    assert h.sage_attn_ref_rows_f32(*bad) == INVALID
    bad = list(args)
    bad[10] = 0                    # nrows
    assert h.sage_attn_ref_rows_f32(*bad) == INVALID
    bad = list(args)
    bad[7] = 96                    # d
    assert h.sage_attn_ref_rows_f32(*bad) == UNSUPPORTED
    if not torch.cuda.is_available():
        assert h.sage_attn_ref_rows_f32(*args) == NO_DEVICE


def test_layout_and_rope_validation():
    h = lib()
    ws = P + 0x100000
    base = [P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 0, 0]
    # layout, rope_cos, rope_sin, out_f32, workspace, bytes, stream
    assert h.sage_attn_fwd_ex(*base, 2, None, None, 0, ws, 1 << 40, None) == INVALID
    assert h.sage_attn_fwd_ex(*base, 1, P, None, 0, ws, 1 << 40, None) == INVALID
    assert h.sage_attn_fwd_ex(*base, 1, P + 4, P, 0, ws, 1 << 40, None) == INVALID
    assert h.sage_attn_fwd_ex(*base, 0, None, None, 2, ws, 1 << 40, None) == INVALID
    assert h.sage_smooth_quant_qk_ex(P, P, 0, 3, None, None, 1, 1, 300, 64, P, P, P, P, P, P,
                                     1 << 30, None) == INVALID
    assert h.sage_smooth_quant_qk_ex(P, P, 0, 0, None, P, 1, 1, 300, 64, P, P, P, P, P, P,
                                     1 << 30, None) == INVALID
    assert h.sage_quant_v_ex(P, 0, 5, 1, 1, 300, 64, 0, P, None, P, 1 << 30, None) == INVALID
    if not torch.cuda.is_available():
        assert h.sage_attn_fwd_ex(*base, 1, P, P, 1, ws, 1 << 40, None) == NO_DEVICE
        assert h.sage_smooth_quant_qk_ex(P, P, 0, 1, P, P, 1, 1, 300, 64, P, P, P, P, P, P,
                                         1 << 30, None) == NO_DEVICE
        assert h.sage_quant_v_ex(P, 0, 1, 1, 1, 300, 64, 0, P, None, P, 1 << 30, None) == NO_DEVICE


def test_smooth_q_workspace_chunks():
    """The smoothed-Q seed table: int32 values for ceil(N/64)*64 keys per head
    and 128-row query block, all blocks while that stays within 256 MiB, else
    an even number of blocks per chunk (at least two).  The difference between
    the two workspace sizes is that table plus q-bar and w (2 x d x 4 bytes per
    block and head) and their 256-byte slice alignment."""
    h = lib()
    MiB = 1 << 20

    def table(B, H, N, d):
        return h.sage_attn_sq_workspace_bytes(B, H, N, d, 0) - h.sage_attn_workspace_bytes(B, H, N, d, 0)

    def expect(B, H, N, d, blocks):
        nt64 = -(-N // 64) * 64
        extra = B * H * blocks * nt64 * 4 + 2 * B * H * (-(-N // 128)) * d * 4
        return extra

    # c3's shape: one chunk, 201 MB of seeds
    assert abs(table(1, 24, 16384, 128) - expect(1, 24, 16384, 128, 128)) <= 3 * 256
    # one head of 2^17 tokens: 1024 blocks of 512 KiB would be 512 MiB -> 512 per chunk
    assert abs(table(1, 1, 1 << 17, 128) - expect(1, 1, 1 << 17, 128, 512)) <= 3 * 256
    # 2^17 + 17 tokens: 2049 key tiles, 256 MiB holds 511 blocks -> 510 (even)
    assert abs(table(1, 1, (1 << 17) + 17, 128) - expect(1, 1, (1 << 17) + 17, 128, 510)) <= 3 * 256
    assert table(1, 1, (1 << 17) + 17, 128) < 260 * MiB
    # many heads at a long N: one block of every head exceeds 256 MiB -> two per chunk
    assert abs(table(4, 32, 1 << 20, 64) - expect(4, 32, 1 << 20, 64, 2)) <= 3 * 256


def test_smooth_q_entries_validation():
    # sage_attn_fwd_sq: q, k, v, o, B, H, N, d, causal, pv, dtype, layout, out_f32, ws, bytes, stream
    h = lib()
    ws = P + 0x100000
    need = h.sage_attn_sq_workspace_bytes(1, 2, 100, 64, 0)
    assert need > h.sage_attn_workspace_bytes(1, 2, 100, 64, 0)   # + means, w, compensation
    assert h.sage_attn_sq_workspace_bytes(1, 2, 100, 96, 0) == 0
    assert h.sage_attn_sq_workspace_bytes(1, 2, 100, 64, 3) == 0
    base = [P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 0, 0]
    assert h.sage_attn_fwd_sq(*base, 0, 2, ws, 1 << 40, None) == INVALID        # out_f32
    assert h.sage_attn_fwd_sq(*base, 2, 0, ws, 1 << 40, None) == INVALID        # layout
    assert h.sage_attn_fwd_sq(*base, 0, 0, ws, need - 1, None) == WORKSPACE
    assert h.sage_attn_fwd_sq(P, P, P, P, *base[4:], 0, 0, ws, 1 << 40, None) == INVALID  # o aliases q
    if not torch.cuda.is_available():
        assert h.sage_attn_fwd_sq(*base, 0, 0, ws, need, None) == NO_DEVICE
    # sage_smooth_q: q, k_i8, dtype, B, H, N, d, seed_pv_mode, q_i8, q_scale, q_mean, q_w, q_comp
    args = [P, P, 0, 1, 2, 100, 64, -1, P, P, P, P, P, None]
    bad = list(args)
    bad[7] = 5                      # seed mode
    assert h.sage_smooth_q(*bad) == INVALID
    bad = list(args)
    bad[12] = P + 4                 # q_comp not 16-byte aligned
    assert h.sage_smooth_q(*bad) == INVALID
    bad = list(args)
    bad[6] = 96
    assert h.sage_smooth_q(*bad) == UNSUPPORTED
    # sage_attn_fwd_quantized_sq: the seeds are required and 16-byte aligned
    qargs = [P] * 6 + [P, P] + [1, 2, 100, 64, 0, 0, 0, None]
    bad = list(qargs)
    bad[6] = None
    assert h.sage_attn_fwd_quantized_sq(*bad) == INVALID
    bad = list(qargs)
    bad[6] = P + 8
    assert h.sage_attn_fwd_quantized_sq(*bad) == INVALID
    if not torch.cuda.is_available():
        assert h.sage_smooth_q(*args) == NO_DEVICE
        assert h.sage_attn_fwd_quantized_sq(*qargs) == NO_DEVICE


def test_prepare_validation():
    # q, k, v, B, H, N, d, pv, dtype, workspace, bytes, stream
    h = lib()
    ws = P + 0x100000
    need = h.sage_attn_workspace_bytes(1, 2, 100, 64, 0)
    base = [P, P + 0x1000, P + 0x2000, 1, 2, 100, 64, 0, 0, ws, need, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return h.sage_attn_prepare(*a)
    assert call(a0=None) == INVALID
    assert call(a2=P + 4) == INVALID            # v not 16-byte aligned
    assert call(a9=P + 16) == INVALID           # workspace not 256-byte aligned
    assert call(a7=3) == INVALID
    assert call(a8=2) == INVALID
    assert call(a5=0) == INVALID
    assert call(a6=96) == UNSUPPORTED
    assert call(a5=(1 << 24) + 1) == UNSUPPORTED
    assert call(a10=need - 1) == WORKSPACE
    if not torch.cuda.is_available():
        assert call() == NO_DEVICE


def test_attend_validation():
    # workspace, bytes, o, B, H, N, d, causal, pv, out_dtype, stream
    h = lib()
    ws = P + 0x100000
    need = h.sage_attn_workspace_bytes(1, 2, 100, 64, 1)
    base = [ws, need, P, 1, 2, 100, 64, 0, 1, 0, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return h.sage_attn_attend(*a)
    assert call(a0=None) == INVALID
    assert call(a2=None) == INVALID
    assert call(a2=P + 8) == INVALID            # o not 16-byte aligned
    assert call(a0=ws + 16) == INVALID          # workspace not 256-byte aligned
    assert call(a7=2) == INVALID                # causal flag
    assert call(a8=3) == INVALID                # P~V mode
    assert call(a9=3) == INVALID                # output type
    assert call(a4=0) == INVALID
    assert call(a6=96) == UNSUPPORTED
    assert call(a5=(1 << 24) + 1) == UNSUPPORTED
    assert call(a1=need - 1) == WORKSPACE
    if not torch.cuda.is_available():
        assert call() == NO_DEVICE
        assert call(a9=2) == NO_DEVICE          # float32 output is a valid type


def test_debug_s_fwd_validation():
    # workspace, bytes, B, H, N, d, causal, pv, smooth_q, b, h, q0, nq, k0, nk, s_out, o_rows, stream
    h = lib()
    ws = P + 0x100000
    need = h.sage_attn_workspace_bytes(1, 2, 100, 64, 0)
    need_sq = h.sage_attn_sq_workspace_bytes(1, 2, 100, 64, 0)
    args = [ws, need, 1, 2, 100, 64, 0, 0, 0, 0, 1, 0, 100, 0, 100, P, P + 0x1000, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return h.sage_attn_debug_s_fwd(*a)
    assert call(a0=None) == INVALID
    assert call(a0=P + 16) == INVALID           # workspace not 256-byte aligned
    assert call(a15=None) == INVALID
    assert call(a16=P + 4) == INVALID           # o_rows not 16-byte aligned
    assert call(a6=2) == INVALID
    assert call(a8=2) == INVALID
    assert call(a7=3) == INVALID
    assert call(a10=2) == INVALID               # head out of range
    assert call(a11=100) == INVALID             # q0 >= N
    assert call(a12=101) == INVALID             # window past N
    assert call(a13=-1) == INVALID
    assert call(a14=0) == INVALID
    assert call(a5=96) == UNSUPPORTED
    assert call(a1=need - 1) == WORKSPACE
    assert call(a8=1, a1=need) == WORKSPACE     # Q smoothed needs the larger workspace
    # Q smoothed on a head whose seed table took more than one chunk: the
    # workspace holds the last chunk only, so the scores cannot be rebuilt
    NL = (1 << 17) + 17
    need_long = h.sage_attn_sq_workspace_bytes(1, 1, NL, 128, 0)
    assert h.sage_attn_debug_s_fwd(ws, need_long, 1, 1, NL, 128, 0, 0, 1, 0, 0, 0, 128, 0, 64,
                                   P, P + 0x1000, None) == UNSUPPORTED
    if not torch.cuda.is_available():
        assert call() == NO_DEVICE
        assert call(a8=1, a1=need_sq) == NO_DEVICE
        assert h.sage_attn_debug_fwd_f32(P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 0, 0,
                                         P + 0x100000, 1 << 40, None) == NO_DEVICE


def test_sequence_length_limit():
    # the documented limit 2^24 tokens is accepted, one more is not (the
    # kernels' 32-bit buffer offsets are sized for it: static_asserts in the
    # attention kernel's source)
    h = lib()
    assert "N <= 2^24" in open(HEADER).read()
    for pv in (0, 1, 2):
        for d in (64, 128):
            assert h.sage_attn_workspace_bytes(1, 1, 1 << 24, d, pv) > (1 << 24) * d * 2
            assert h.sage_attn_workspace_bytes(1, 1, (1 << 24) + 1, d, pv) == 0
    assert fwd(N=1 << 24, d=128, wsb=1000) == WORKSPACE    # shape accepted, workspace checked


def test_probe_library_exports():
    from quantized_attention_qk_amd import probe
    src = open(os.path.join(ROOT, "include", "sage_probe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))
    assert names == ["sage_probe_cu_count", "sage_probe_run", "sage_probe_run_lds",
                     "sage_probe_wallclock_khz"]
    h = probe.lib()
    for n in names:
        assert hasattr(h, n), n
    # invalid arguments are rejected before any launch
    assert h.sage_probe_run(0, 0, 0, 3, 256, 1024, P, P, None) == 1
    assert h.sage_probe_run(0, 0, 0, 2, 256, 1023, P, P, None) == 1
    assert h.sage_probe_run(5, 0, 0, 2, 256, 1024, P, P, None) == 1
    assert h.sage_probe_run_lds(1, 1, 3, 256, 1024, P, P, None) == 1
    assert h.sage_probe_run_lds(1, 1, 2, 256, 1022, P, P, None) == 1
    assert h.sage_probe_run_lds(7, 1, 2, 256, 1024, P, P, None) == 1
    assert h.sage_probe_run_lds(1, 3, 2, 256, 1024, P, P, None) == 2   # nl not 1, 2, 4


def test_noalloc_validation():
    # q, k, v, o, B, H, N, d, causal, pv_mode, dtype, stream
    h = lib()
    assert h.sage_attn_fwd_noalloc(P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 3, 0, None) == INVALID
    assert h.sage_attn_fwd_noalloc(P, P, P, P + 0x1000, 0, 2, 100, 64, 0, 0, 0, None) == INVALID
    assert h.sage_attn_fwd_noalloc(P, P, P, P + 0x1000, 1, 2, 100, 96, 0, 0, 0, None) == UNSUPPORTED
    # beyond the fixed workspace (c3's shape needs about 200 MB)
    assert h.sage_attn_workspace_bytes(1, 24, 16384, 128, 0) > (128 << 20)
    assert h.sage_attn_fwd_noalloc(P, P, P, P + 0x1000, 1, 24, 16384, 128, 0, 0, 1,
                                   None) == WORKSPACE
    assert "#define SAGE_NOALLOC_MAX_WORKSPACE ((size_t)128 << 20)" in open(HEADER).read()
    if not torch.cuda.is_available():
        assert h.sage_attn_fwd_noalloc(P, P, P, P + 0x1000, 1, 2, 100, 64, 0, 0, 0,
                                       None) == NO_DEVICE
