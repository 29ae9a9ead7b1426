"""Python entry points over the C ABI (argument marshalling only).

Every step of the forward pass runs in the HIP kernels of libsage_attn.so;
torch provides device memory (outputs, workspace) and the current stream.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import SAGE_DT, SAGE_LAYOUT, SAGE_PV, check, lib

__all__ = ["sage_attn", "sage_attn_quantized", "ref_rows", "smooth_quant_qk", "quant_v", "debug_s_i32",
           "debug_s_fwd", "tiling", "workspace_bytes", "untile_v"]


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_qkv(*ts, layout: str = "HND"):
    """(B, H, N, d) of contiguous 16-bit device tensors in `layout`
    ("HND": [B, H, N, d]; "NHD": [B, N, H, d])."""
    if layout not in SAGE_LAYOUT:
        raise ValueError(f"layout {layout!r} (HND or NHD)")
    q = ts[0]
    if q.dim() != 4:
        raise ValueError("expected 4-d tensors")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if t.dtype not in SAGE_DT:
            raise ValueError(f"dtype {t.dtype} not supported (float16 or bfloat16)")
        if t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k, v must share dtype, shape and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if layout == "HND":
        return tuple(q.shape)
    B, N, H, d = q.shape
    return B, H, N, d


def _rope_ptrs(rope, N, d, dev):
    """Device pointers of float32 [N, d/2] cos/sin tables, or (None, None)."""
    if rope is None:
        return None, None, ()
    cos, sin = rope
    for t in (cos, sin):
        if (not t.is_cuda or t.device != dev or t.dtype != torch.float32 or
                tuple(t.shape) != (N, d // 2) or not t.is_contiguous()):
            raise ValueError("rope tables must be contiguous float32 [N, d/2] on the device")
    return cos.data_ptr(), sin.data_ptr(), (cos, sin)


def tiling(d: int = 128, causal: bool = False, pv_mode: str = "fp16") -> dict:
    vals = [ctypes.c_int() for _ in range(4)]
    check(lib().sage_attn_get_tiling(d, int(causal), SAGE_PV[pv_mode], *[ctypes.byref(v) for v in vals]),
          "sage_attn_get_tiling")
    return dict(zip(("q_block", "k_block", "kv_tile", "mean_chunk"), (v.value for v in vals)))


def workspace_bytes(B: int, H: int, N: int, d: int, pv_mode: str = "fp16",
                    smooth_q: bool = False) -> int:
    if smooth_q:
        return int(lib().sage_attn_sq_workspace_bytes(B, H, N, d, SAGE_PV[pv_mode]))
    return int(lib().sage_attn_workspace_bytes(B, H, N, d, SAGE_PV[pv_mode]))


def sage_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
              pv_mode: str = "fp16", out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, out_f32: bool = False,
              layout: str = "HND", rope=None, smooth_q: bool = False) -> torch.Tensor:
    """SageAttention forward: O = softmax(Q K^T / sqrt(d)) V with smoothed INT8
    Q K^T and FP16, FP8 or INT8 P~V.  q, k, v: contiguous fp16/bf16 tensors, [B, H, N,
    d] (layout "HND") or [B, N, H, d] ("NHD"); O has the same layout.

    rope: optional (cos, sin) float32 [N, d/2] device tables; Q and K are then
    rotated (rotate-half form) inside the quantisation prepass.
    smooth_q: smooth Q per 128-token block as well as K (sage_attn_fwd_sq);
    not combined with rope.
    Returns O in the input dtype, or float32 when `out_f32`.  `workspace` may
    be a preallocated uint8 device tensor of workspace_bytes(...) bytes.
    """
    B, H, N, d = _check_qkv(q, k, v, layout=layout)
    mode = SAGE_PV[pv_mode]
    if smooth_q and rope is not None:
        raise ValueError("smooth_q is not combined with rope")
    need = workspace_bytes(B, H, N, d, pv_mode, smooth_q)
    if need == 0:
        raise ValueError(f"unsupported shape {(B, H, N, d)}")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    elif out.dtype != odt or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and the output dtype")
    pc, ps, keep = _rope_ptrs(rope, N, d, q.device)
    if smooth_q:
        check(lib().sage_attn_fwd_sq(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                     H, N, d, int(causal), mode, SAGE_DT[q.dtype],
                                     SAGE_LAYOUT[layout], int(out_f32), workspace.data_ptr(),
                                     workspace.numel(), _stream_ptr(q.device)),
              "sage_attn_fwd_sq")
    elif layout == "HND" and rope is None:
        fn = lib().sage_attn_fwd_f32out if out_f32 else lib().sage_attn_fwd
        check(fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                 int(causal), mode, SAGE_DT[q.dtype], workspace.data_ptr(), workspace.numel(),
                 _stream_ptr(q.device)), "sage_attn_fwd")
    else:
        check(lib().sage_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                     H, N, d, int(causal), mode, SAGE_DT[q.dtype],
                                     SAGE_LAYOUT[layout], pc, ps, int(out_f32),
                                     workspace.data_ptr(), workspace.numel(),
                                     _stream_ptr(q.device)), "sage_attn_fwd_ex")
    del keep
    return out


def smooth_quant_qk(q: torch.Tensor, k: torch.Tensor, layout: str = "HND", rope=None) -> dict:
    """Smooth K and quantise Q/sqrt(d), K to INT8 per block (the prepass), with
    optional RoPE applied first.  Outputs are [B, H, N, d]-ordered."""
    B, H, N, d = _check_qkv(q, k, layout=layout)
    dev = q.device
    nqb, nkb = -(-N // 128), -(-N // 64)
    res = dict(q_i8=torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
               k_i8=torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
               q_scale=torch.empty((B, H, nqb), dtype=torch.float32, device=dev),
               k_scale=torch.empty((B, H, nkb), dtype=torch.float32, device=dev),
               k_mean=torch.empty((B, H, d), dtype=torch.float32, device=dev))
    nscr = int(lib().sage_smooth_quant_qk_scratch_bytes(B, H, N, d))
    scratch = torch.empty(max(nscr, 16), dtype=torch.uint8, device=dev)
    pc, ps, keep = _rope_ptrs(rope, N, d, dev)
    check(lib().sage_smooth_quant_qk_ex(
        q.data_ptr(), k.data_ptr(), SAGE_DT[q.dtype], SAGE_LAYOUT[layout], pc, ps, B, H, N, d,
        res["q_i8"].data_ptr(), res["k_i8"].data_ptr(), res["q_scale"].data_ptr(),
        res["k_scale"].data_ptr(), res["k_mean"].data_ptr(), scratch.data_ptr(), scratch.numel(),
        _stream_ptr(dev)), "sage_smooth_quant_qk_ex")
    del keep
    return res


def smooth_q(q: torch.Tensor, k_i8: torch.Tensor, seed_pv_mode: str | None = None) -> dict:
    """The smoothed-Q stage (sage_smooth_q) on [B,H,N,d] q and the K^ codes of
    smooth_quant_qk: q_i8, q_scale, q_mean, q_w and q_comp (C [B,H,nqb,N]; or,
    with seed_pv_mode, the attention kernel's seeds for that P~V mode,
    [B,H,nqb,ceil(N/64)*64], the input of sage_attn_quantized's q_seed)."""
    B, H, N, d = _check_qkv(q)
    dev = q.device
    nqb = -(-N // 128)
    ncomp = N if seed_pv_mode is None else -(-N // 64) * 64
    res = dict(q_i8=torch.empty((B, H, N, d), dtype=torch.int8, device=dev),
               q_scale=torch.empty((B, H, nqb), dtype=torch.float32, device=dev),
               q_mean=torch.empty((B, H, nqb, d), dtype=torch.float32, device=dev),
               q_w=torch.empty((B, H, nqb, d), dtype=torch.int32, device=dev),
               q_comp=torch.empty((B, H, nqb, ncomp), dtype=torch.int32, device=dev))
    if tuple(k_i8.shape) != (B, H, N, d) or k_i8.dtype != torch.int8 or not k_i8.is_contiguous():
        raise ValueError("k_i8 must be a contiguous int8 tensor of q's shape")
    check(lib().sage_smooth_q(q.data_ptr(), k_i8.data_ptr(), SAGE_DT[q.dtype], B, H, N, d,
                              -1 if seed_pv_mode is None else SAGE_PV[seed_pv_mode],
                              res["q_i8"].data_ptr(), res["q_scale"].data_ptr(),
                              res["q_mean"].data_ptr(), res["q_w"].data_ptr(),
                              res["q_comp"].data_ptr(), _stream_ptr(dev)), "sage_smooth_q")
    return res


def quant_v(v: torch.Tensor, pv_mode: str = "fp16", layout: str = "HND"):
    """Prepare V for P~V: (tiled uint8 tensor, per-channel scale or None)."""
    B, H, N, d = _check_qkv(v, layout=layout)
    dev = v.device
    mode = SAGE_PV[pv_mode]
    v_out = torch.empty(int(lib().sage_quant_v_bytes(B, H, N, d, mode)), dtype=torch.uint8,
                        device=dev)
    v_scale = torch.empty((B, H, d), dtype=torch.float32, device=dev) if mode != 0 else None
    nscr = int(lib().sage_quant_v_scratch_bytes(B, H, N, d, mode))
    scratch = torch.empty(max(nscr, 16), dtype=torch.uint8, device=dev)
    check(lib().sage_quant_v_ex(v.data_ptr(), SAGE_DT[v.dtype], SAGE_LAYOUT[layout], B, H, N, d,
                                mode, v_out.data_ptr(),
                                v_scale.data_ptr() if v_scale is not None else None,
                                scratch.data_ptr(), scratch.numel(), _stream_ptr(dev)),
          "sage_quant_v_ex")
    return v_out, v_scale


def sage_attn_quantized(qk: dict, v_prep: torch.Tensor, v_scale: torch.Tensor | None,
                        causal: bool = False, pv_mode: str = "fp16",
                        out_dtype: torch.dtype = torch.bfloat16,
                        out: torch.Tensor | None = None,
                        q_seed: torch.Tensor | None = None) -> torch.Tensor:
    """The attention kernel alone, on the outputs of smooth_quant_qk/quant_v
    (with Q smoothed: q_i8, q_scale from smooth_q and q_seed = its q_comp
    for the same pv_mode)."""
    q_i8 = qk["q_i8"]
    B, H, N, d = q_i8.shape
    odt = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}[out_dtype]
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q_i8.device)
    vsp = v_scale.data_ptr() if v_scale is not None else None
    if q_seed is not None:
        check(lib().sage_attn_fwd_quantized_sq(
            q_i8.data_ptr(), qk["k_i8"].data_ptr(), v_prep.data_ptr(), qk["q_scale"].data_ptr(),
            qk["k_scale"].data_ptr(), vsp, q_seed.data_ptr(), out.data_ptr(), B, H, N, d,
            int(causal), SAGE_PV[pv_mode], odt, _stream_ptr(q_i8.device)),
            "sage_attn_fwd_quantized_sq")
        return out
    check(lib().sage_attn_fwd_quantized(
        q_i8.data_ptr(), qk["k_i8"].data_ptr(), v_prep.data_ptr(), qk["q_scale"].data_ptr(),
        qk["k_scale"].data_ptr(), vsp,
        out.data_ptr(), B, H, N, d, int(causal), SAGE_PV[pv_mode], odt,
        _stream_ptr(q_i8.device)), "sage_attn_fwd_quantized")
    return out


def ref_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rows: torch.Tensor,
             causal: bool = False) -> torch.Tensor:
    """Float32 softmax attention (no quantisation) on the query rows `rows`
    of every (b, h): returns [B, H, len(rows), d] float32."""
    B, H, N, d = _check_qkv(q, k, v)
    rows = rows.to(device=q.device, dtype=torch.int32).contiguous()
    out = torch.empty((B, H, rows.numel(), d), dtype=torch.float32, device=q.device)
    check(lib().sage_attn_ref_rows_f32(q.data_ptr(), k.data_ptr(), v.data_ptr(), SAGE_DT[q.dtype],
                                       B, H, N, d, int(causal), rows.data_ptr(), rows.numel(),
                                       out.data_ptr(), _stream_ptr(q.device)),
          "sage_attn_ref_rows_f32")
    return out


def debug_s_i32(q_i8: torch.Tensor, k_i8: torch.Tensor, b: int, h: int, q0: int, nq: int,
                k0: int, nk: int) -> torch.Tensor:
    """INT32 S = Q^ K^T on a rectangle, by the attention kernel's MFMA code."""
    B, H, N, d = q_i8.shape
    if q_i8.dtype != torch.int8 or k_i8.dtype != torch.int8 or k_i8.shape != q_i8.shape:
        raise ValueError("q_i8, k_i8 must be int8 [B, H, N, d]")
    s = torch.empty((nq, nk), dtype=torch.int32, device=q_i8.device)
    check(lib().sage_attn_debug_s_i32(q_i8.data_ptr(), k_i8.data_ptr(), B, H, N, d, b, h, q0, nq,
                                      k0, nk, s.data_ptr(), _stream_ptr(q_i8.device)),
          "sage_attn_debug_s_i32")
    return s


S_NOT_COMPUTED = -(2 ** 31)   # entries of debug_s_fwd's S the kernel did not compute


def prepare(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, pv_mode: str,
            workspace: torch.Tensor) -> None:
    """The prepass of sage_attn alone (sage_attn_prepare): leaves the quantised
    operands in `workspace` for debug_s_fwd and launches no attention.  q, k, v
    contiguous [B, H, N, d] fp16/bf16 on the GPU."""
    B, H, N, d = _check_qkv(q, k, v)
    check(lib().sage_attn_prepare(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d,
                                  SAGE_PV[pv_mode], SAGE_DT[q.dtype], workspace.data_ptr(),
                                  workspace.numel(), _stream_ptr(q.device)), "sage_attn_prepare")


def attend(workspace: torch.Tensor, B: int, H: int, N: int, d: int, causal: bool = False,
           pv_mode: str = "fp16", out_dtype: torch.dtype = torch.bfloat16,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """The attention kernel of sage_attn alone (sage_attn_attend) on the
    operands a preceding prepare(...) with the same shape and pv_mode left in
    `workspace` (same stream).  prepare + attend = sage_attn, bit for bit."""
    odt = {torch.float16: 0, torch.bfloat16: 1, torch.float32: 2}[out_dtype]
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=workspace.device)
    check(lib().sage_attn_attend(workspace.data_ptr(), workspace.numel(), out.data_ptr(), B, H,
                                 N, d, int(causal), SAGE_PV[pv_mode], odt,
                                 _stream_ptr(workspace.device)), "sage_attn_attend")
    return out


def debug_s_fwd(workspace: torch.Tensor, B: int, H: int, N: int, d: int, causal: bool,
                pv_mode: str, smooth_q: bool, b: int, h: int, q0: int, nq: int, k0: int,
                nk: int):
    """The INT32 scores of the timed attention kernel itself (its debug
    instantiation, re-run on the operands a preceding sage_attn(...,
    workspace=workspace) call left there) for head (b, h), queries [q0, q0+nq)
    and keys [k0, k0+nk): returns (S int32 [nq, nk] with S_NOT_COMPUTED where
    the kernel computes no score, O float32 [nq, d] of those rows)."""
    dev = workspace.device
    s = torch.full((nq, nk), S_NOT_COMPUTED, dtype=torch.int32, device=dev)
    o = torch.full((nq, d), float("nan"), dtype=torch.float32, device=dev)
    check(lib().sage_attn_debug_s_fwd(workspace.data_ptr(), workspace.numel(), B, H, N, d,
                                      int(causal), SAGE_PV[pv_mode], int(smooth_q), b, h, q0, nq,
                                      k0, nk, s.data_ptr(), o.data_ptr(), _stream_ptr(dev)),
          "sage_attn_debug_s_fwd")
    return s, o


def untile_v(v_out, B: int, H: int, N: int, d: int, pv_mode: str = "fp16"):
    """Inverse of the tiled V layout documented for sage_quant_v: returns a
    numpy array [B, H, N, d] (float16 values, uint8 E4M3 codes or int8
    codes)."""
    import numpy as np
    raw = v_out.cpu().numpy() if hasattr(v_out, "cpu") else np.asarray(v_out)
    nt = -(-N // 64)
    c = np.arange(d)[:, None]
    if pv_mode == "fp16":
        t = raw.view(np.float16).reshape(B, H, nt, d, 8, 8)      # [.., c, phys chunk, e]
        kk = np.arange(8)[None, :] ^ ((c // 2) % 8)              # logical chunk of each phys chunk
        e = np.arange(8)
        key = 16 * (kk[:, :, None] // 2) + 8 * (e // 4) + 4 * (kk[:, :, None] % 2) + e % 4
        out = np.zeros((B, H, nt, 64, d), np.float16)
        cc = np.broadcast_to(c[:, :, None], key.shape)
        out[:, :, :, key, cc] = t
    else:
        t = raw.reshape(B, H, nt, d, 4, 16)
        lq = np.arange(4)[None, :] ^ ((c // 4) % 4)
        p = 16 * lq[:, :, None] + np.arange(16)
        key = 32 * ((p // 16) % 2) + 8 * ((p % 16) // 4) + 4 * (p // 32) + p % 4
        out = np.zeros((B, H, nt, 64, d), np.uint8)
        cc = np.broadcast_to(c[:, :, None], key.shape)
        out[:, :, :, key, cc] = t
        if pv_mode == "int8":
            out = out.view(np.int8)
    return out.reshape(B, H, nt * 64, d)[:, :, :N]
