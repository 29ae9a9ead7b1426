"""GPU parity of the fused RoPE + quantisation prepass and of the token-major
[B, N, H, d] layout ("SageAttention ..." detail page, §7 key implementation
details, item 1: Q and K are quantised in the kernel that applies RoPE).

Bar: the prepass (K mean of the rotated K, delta_Q, delta_K, Q^, K^, V') is
bit-exact against the oracle applied to the rotated inputs; O (float32) within
max-abs 2e-3 and cosine >= 0.9999; without RoPE the token-major layout gives
bit-identical O to the [B, H, N, d] layout.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, rope_tables, small, to_nhd

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-3
O_COS = 0.9999


def note(msg):
    print(f"[gpu-rope] {msg}", flush=True)
    sys.stdout.flush()


def qa():
    import quantized_attention_qk_amd as m
    return m


def to_np(t):
    return t.detach().cpu().numpy()


def dev_inputs(inp, layout):
    q, k, v = inp.torch_tensors("cpu")
    if layout == "NHD":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    return q.cuda(), k.cuda(), v.cuda()


def dev_rope(N, d, offset=0):
    c, s = rope_tables(N, d, offset=offset)
    return (torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda()), (c, s)


CASES = [
    small("r65", N=65, d=64, dtype="fp16"),
    small("r197c8", N=197, d=64, causal=True, pv_mode="fp8"),
    small("r300", B=2, H=3, N=300, d=128, dtype="bf16", extras="q8_kbias5"),
    small("r640c8", N=640, d=128, causal=True, dtype="bf16", pv_mode="fp8", extras="kchan20"),
    small("r2113c8", N=2113, d=64, pv_mode="fp8", extras="kbias4"),
    small("r300i8", B=2, H=3, N=300, d=128, dtype="bf16", pv_mode="int8", extras="q8_kbias5"),
    small("r2113ci8", N=2113, d=64, causal=True, pv_mode="int8", extras="kbias4"),
]


def assert_prepass(res, pq, what):
    g = {k: to_np(t) for k, t in res.items()}
    for key in ("k_mean", "q_scale", "k_scale"):
        np.testing.assert_array_equal(g[key].view(np.uint32), pq[key].view(np.uint32),
                                      err_msg=f"{what} {key} bits")
    np.testing.assert_array_equal(g["q_i8"], pq["q_i8"], err_msg=f"{what} q_i8")
    np.testing.assert_array_equal(g["k_i8"], pq["k_i8"], err_msg=f"{what} k_i8")


@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_rope_prepass_bit_exact(wl, layout):
    note(f"rope prepass {wl.name} {layout}")
    inp = make_inputs(wl)
    q, k, v = dev_inputs(inp, layout)
    rope_d, (c, s) = dev_rope(wl.N, wl.d, offset=7)
    res = qa().smooth_quant_qk(q, k, layout=layout, rope=rope_d)
    vt_l, vs_l = qa().quant_v(v, wl.pv_mode, layout=layout)
    qh, kh, vh = inp.torch_tensors("cuda")
    vt_h, vs_h = qa().quant_v(vh, wl.pv_mode)
    torch.cuda.synchronize()
    pq = oracle.smooth_quant_qk(oracle.rope_rotate_half(inp.qf, c, s),
                                oracle.rope_rotate_half(inp.kf, c, s))
    assert_prepass(res, pq, f"{wl.name} {layout}")
    assert torch.equal(vt_l, vt_h), "V' of the two layouts"
    if vs_l is not None:
        assert torch.equal(vs_l, vs_h), "delta_V of the two layouts"


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_nhd_layout_bit_identical_without_rope(wl):
    note(f"layout identity {wl.name}")
    inp = make_inputs(wl)
    qh, kh, vh = dev_inputs(inp, "HND")
    qn, kn, vn = dev_inputs(inp, "NHD")
    oh = qa().sage_attn(qh, kh, vh, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    on = qa().sage_attn(qn, kn, vn, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                        layout="NHD")
    torch.cuda.synchronize()
    assert torch.equal(on.transpose(1, 2), oh)


@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_rope_forward_parity(wl, layout):
    note(f"rope forward {wl.name} {layout}")
    inp = make_inputs(wl)
    q, k, v = dev_inputs(inp, layout)
    rope_d, (c, s) = dev_rope(wl.N, wl.d)
    o = to_np(qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                             layout=layout, rope=rope_d))
    if layout == "NHD":
        o = np.swapaxes(o, 1, 2)
    ref = oracle.sage_attention(oracle.rope_rotate_half(inp.qf, c, s),
                                oracle.rope_rotate_half(inp.kf, c, s), inp.vf,
                                causal=wl.causal, pv_mode=wl.pv_mode)
    err = np.abs(o.astype(np.float64) - ref)
    cos = oracle.cos_sim(o, ref)
    note(f"{wl.name} {layout}: max|dO| = {err.max():.3e} cos = {cos:.7f}")
    assert err.max() <= O_MAX_ABS and cos >= O_COS


def test_rope_nhd_full_size_sampled_rows():
    # the c2 shape (LLM prefill: B=4, H=32, N=4096, d=128, causal, bf16), with
    # RoPE and token-major inputs; prepass bit-exact on two heads, O on rows
    wl = WORKLOADS["c2"]
    note(f"full size rope + NHD {wl}")
    inp = make_inputs(wl)
    q, k, v = dev_inputs(inp, "NHD")
    rope_d, (c, s) = dev_rope(wl.N, wl.d)
    res = qa().smooth_quant_qk(q, k, layout="NHD", rope=rope_d)
    o = qa().sage_attn(q, k, v, causal=True, pv_mode="fp16", out_f32=True, layout="NHD",
                       rope=rope_d)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 2047, 4094, 4095} |
                           set(int(x) for x in np.random.default_rng(5).integers(0, 4096, 12))))
    for (b, h) in [(0, 0), (3, 31)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        qr = oracle.rope_rotate_half(inp.qf[sl], c, s)
        kr = oracle.rope_rotate_half(inp.kf[sl], c, s)
        pq = oracle.smooth_quant_qk(qr, kr)
        g = {key: to_np(t)[b:b + 1, h:h + 1] for key, t in res.items()}
        for key in ("k_mean", "q_scale", "k_scale"):
            np.testing.assert_array_equal(g[key].view(np.uint32), pq[key].view(np.uint32))
        np.testing.assert_array_equal(g["q_i8"], pq["q_i8"])
        np.testing.assert_array_equal(g["k_i8"], pq["k_i8"])
        ref = oracle.sage_attention(qr, kr, inp.vf[sl], causal=True, pv_mode="fp16",
                                    rows=rows)[0, 0]
        got = to_np(o[b, torch.from_numpy(rows).cuda(), h])
        err = np.abs(got.astype(np.float64) - ref)
        note(f"(b={b},h={h}): max|dO| = {err.max():.3e}")
        assert err.max() <= O_MAX_ABS and oracle.cos_sim(got, ref) >= O_COS
