"""GPU parity of the smoothed-Q path (Q smoothed per 128-token block as well
as K, the SageAttention2 step; reading documented in include/sage_attn.h and
the oracle's module docstring).

* the stage sage_smooth_q against the oracle, bit for bit: Q~^ codes, delta_Q,
  the block means, the integer means w, the compensation C (and the attention
  kernel's seeds, C plus FP16 mode's accumulator bias), including a block that
  the guard leaves unsmoothed;
* the whole pass (sage_attn_fwd_sq) against the oracle's O, in the three P~V
  modes, to the bar of test_gpu_parity.py;
* the stage-wise path equals the whole pass bit for bit;
* full-size shapes on sampled rows; on a Q with a per-channel bias shared by
  all tokens the smoothed pass is closer to exact attention.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs, named, small

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-3
O_COS = 0.9999


def note(msg):
    print(f"[gpu-smooth-q] {msg}", flush=True)
    sys.stdout.flush()


def qa():
    import quantized_attention_qk_amd as m
    return m


def to_np(t):
    return t.detach().cpu().numpy()


def guard_inputs(wl):
    """The workload's inputs with query block 0 of every head moved to
    50 + (fp16-rounded) noise of a few ulps: its mean dwarfs its spread, so
    127 sum|w| exceeds 2^29 and the block must stay unsmoothed."""
    inp = make_inputs(wl)
    rng = np.random.default_rng(99)
    q = inp.qf.copy()
    q[:, :, :128] = 50.0 + 0.03 * rng.integers(-3, 4, size=q[:, :, :128].shape)
    if wl.dtype == "fp16":
        q16 = q.astype(np.float16)
        qt = torch.from_numpy(q16).cuda()
        qf = q16.astype(np.float32)
    else:
        from workloads import bf16_bits_to_f32, round_to_bf16_bits
        bits = round_to_bf16_bits(q)
        qt = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        qf = bf16_bits_to_f32(bits)
    _, k, v = inp.torch_tensors("cuda")
    return qf, inp.kf, inp.vf, qt, k, v


STAGE = [
    small("sq300", N=300, d=64, extras="qbias4_kbias4"),
    small("sq2113", B=1, H=2, N=2113, d=128, dtype="bf16", extras="qbias4_kbias4"),
    small("sq197", N=197, d=64, extras="kbias4"),
    small("sq640c", B=2, H=3, N=640, d=128, dtype="bf16", causal=True, extras="q8_kbias5"),
]


@pytest.mark.parametrize("guard", [False, True])
@pytest.mark.parametrize("wl", STAGE, ids=lambda w: w.name)
def test_smooth_q_stage_bit_exact(wl, guard):
    note(f"stage {wl} guard={guard}")
    if guard:
        qf, kf, vf, q, k, v = guard_inputs(wl)
    else:
        inp = make_inputs(wl)
        qf, kf = inp.qf, inp.kf
        q, k, v = inp.torch_tensors("cuda")
    res = qa().smooth_quant_qk(q, k)
    sq = qa().smooth_q(q, res["k_i8"])
    seeds = {m: qa().smooth_q(q, res["k_i8"], seed_pv_mode=m)["q_comp"] for m in ("fp16", "int8")}
    torch.cuda.synchronize()
    pq = oracle.smooth_quant_qk(qf, kf, smooth_q=True)
    if guard:
        assert not pq["q_smoothed"][:, :, 0].any() and pq["q_smoothed"][:, :, 1:].all()
    g = {key: to_np(t) for key, t in sq.items()}
    np.testing.assert_array_equal(to_np(res["k_i8"]), pq["k_i8"], err_msg="k_i8")
    np.testing.assert_array_equal(g["q_i8"], pq["q_i8"], err_msg="smoothed Q codes")
    for key in ("q_scale", "q_mean"):
        np.testing.assert_array_equal(g[key].view(np.uint32), pq[key].view(np.uint32),
                                      err_msg=f"{key} bits")
    np.testing.assert_array_equal(g["q_w"], pq["q_w"], err_msg="w")
    np.testing.assert_array_equal(g["q_comp"], pq["q_comp"], err_msg="C")
    N = wl.N
    s16, s8 = to_np(seeds["fp16"]), to_np(seeds["int8"])
    biased = (pq["q_comp"].astype(np.int64) + 0x4B400000).astype(np.int32)
    np.testing.assert_array_equal(s16[..., :N], biased, err_msg="FP16 seeds")
    np.testing.assert_array_equal(s8[..., :N], pq["q_comp"], err_msg="INT8 seeds")
    assert np.all(s16[..., N:] == 0x4B400000) and np.all(s8[..., N:] == 0)
    note(f"{wl.name}: smoothed blocks {int(pq['q_smoothed'].sum())}/{pq['q_smoothed'].size}, "
         f"max|C| {int(np.abs(pq['q_comp']).max())}")


def oracle_o(wl, qf, kf, vf, **kw):
    if wl.pv_mode in ("fp8", "int8"):
        return oracle.sage_attention(qf, kf, vf, causal=wl.causal, pv_mode=wl.pv_mode,
                                     smooth_q=True, p_flip=True, **kw)
    return oracle.sage_attention(qf, kf, vf, causal=wl.causal, pv_mode=wl.pv_mode,
                                 smooth_q=True, **kw), None


def compare(o_gpu, ref, allow, what):
    err = np.abs(o_gpu.astype(np.float64) - ref)
    cos = oracle.cos_sim(o_gpu, ref)
    lim = O_MAX_ABS + (0.0 if allow is None else allow)
    note(f"{what}: max|dO| = {err.max():.3e}  cos = {cos:.7f}  beyond 2e-3: "
         f"{int((err > O_MAX_ABS).sum())}")
    assert np.all(err <= lim), f"{what}: max excess {float((err - lim).max())}"
    assert cos >= O_COS, f"{what}: cos {cos}"


FWD = [
    small("f300", N=300, d=64, extras="qbias4_kbias4"),
    small("f1000c", N=1000, d=128, dtype="bf16", causal=True, extras="qbias4_kbias4"),
    small("f2113", B=1, H=2, N=2113, d=64, extras="qbias4_kbias4"),
    small("f640f8", B=2, H=3, N=640, d=128, dtype="bf16", pv_mode="fp8", extras="qbias4_kbias4"),
    small("f700ci8", N=700, d=64, causal=True, pv_mode="int8", extras="qbias4_kbias4"),
    small("f1500r", N=1500, d=128, extras="ramp"),
    # FP16 P~V at d = 128, non-causal: 256-row workgroups whose second
    # delta_Q block is short (its compensation values sit second in each slot)
    small("f300w", N=300, d=128, dtype="bf16", extras="qbias4_kbias4"),
    small("f129w", N=129, d=128, extras="qbias4_kbias4"),
]


@pytest.mark.parametrize("wl", FWD, ids=lambda w: w.name)
def test_smooth_q_forward_parity(wl):
    note(f"forward {wl}")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    o32 = to_np(qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                               smooth_q=True))
    ref, allow = oracle_o(wl, inp.qf, inp.kf, inp.vf)
    compare(o32, ref, allow, f"{wl.name} O f32")


@pytest.mark.parametrize("wl", [FWD[0], FWD[3], FWD[4]], ids=lambda w: w.name)
def test_smooth_q_guard_block_forward(wl):
    qf, kf, vf, q, k, v = guard_inputs(wl)
    note(f"guard forward {wl.name}")
    o32 = to_np(qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                               smooth_q=True))
    ref, allow = oracle_o(wl, qf, kf, vf)
    compare(o32, ref, allow, f"{wl.name} guard O f32")


@pytest.mark.parametrize("wl", [FWD[1], FWD[3], FWD[4]], ids=lambda w: w.name)
def test_smooth_q_stages_equal_whole_pass(wl):
    note(f"stages {wl.name}")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    whole = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                           smooth_q=True)
    qk = qa().smooth_quant_qk(q, k)
    sq = qa().smooth_q(q, qk["k_i8"], seed_pv_mode=wl.pv_mode)
    qk = dict(qk, q_i8=sq["q_i8"], q_scale=sq["q_scale"])
    vp, vs = qa().quant_v(v, wl.pv_mode)
    staged = qa().sage_attn_quantized(qk, vp, vs, causal=wl.causal, pv_mode=wl.pv_mode,
                                      out_dtype=torch.float32, q_seed=sq["q_comp"])
    torch.cuda.synchronize()
    assert torch.equal(staged.view(torch.int32), whole.view(torch.int32))


@pytest.mark.parametrize("wl", [small("e1", N=1, d=64, extras="qbias4_kbias4"),
                                small("e65", N=65, d=128, dtype="bf16", causal=True,
                                      pv_mode="fp8", extras="qbias4_kbias4"),
                                small("e129i8", N=129, d=64, pv_mode="int8",
                                      extras="qbias4_kbias4")],
                         ids=lambda w: w.name)
def test_smooth_q_edge_lengths(wl):
    # one token (a single-token block: Q~ = 0, so the block stays unsmoothed),
    # a 65-token block, a 1-token last block
    note(f"edge {wl}")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    res = qa().smooth_quant_qk(q, k)
    sq = qa().smooth_q(q, res["k_i8"])
    o32 = to_np(qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                               smooth_q=True))
    torch.cuda.synchronize()
    pq = oracle.smooth_quant_qk(inp.qf, inp.kf, smooth_q=True)
    for key in ("q_i8", "q_w", "q_comp"):
        np.testing.assert_array_equal(to_np(sq[key]), pq[key], err_msg=key)
    np.testing.assert_array_equal(to_np(sq["q_scale"]).view(np.uint32),
                                  pq["q_scale"].view(np.uint32))
    if wl.N == 1:
        assert not pq["q_smoothed"].any()
    ref, allow = oracle_o(wl, inp.qf, inp.kf, inp.vf)
    compare(o32, ref, allow, f"{wl.name} O f32")


@pytest.mark.parametrize("wl", [
    small("sqlong", B=1, H=1, N=(1 << 17) + 17, d=128, dtype="bf16", causal=True,
          extras="qbias4_kbias4", seed=34),
    small("sqlongnc", B=1, H=1, N=(1 << 17) + 17, d=128, dtype="bf16",
          extras="qbias4_kbias4", seed=35),
    small("sqlongf8", B=1, H=1, N=(1 << 17) + 17, d=64, pv_mode="fp8",
          extras="qbias4_kbias4", seed=36),
], ids=lambda w: w.name)
def test_smooth_q_long_head(wl):
    # one head of 2^17 + 17 tokens: its compensation table would be 1025
    # blocks x 131136 keys (512 MiB); the pass runs it in chunks of 510
    # blocks (255 MiB at most), so the workspace stays under 400 MB.  O on
    # rows on both sides of the chunk boundaries (rows 65280 and 130560).
    note(f"long {wl}")
    N = wl.N
    ws = qa().workspace_bytes(1, 1, N, wl.d, wl.pv_mode, smooth_q=True)
    note(f"  workspace {ws / 2**20:.0f} MiB")
    assert ws < 400 * 2**20
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    o32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                         smooth_q=True)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 65279, 65280, 65536, 130559, 130560, N - 18,
                            N - 17, N - 1}))
    ref, allow = oracle_o(wl, inp.qf, inp.kf, inp.vf, rows=rows)
    compare(to_np(o32[0, 0, torch.from_numpy(rows).cuda()]), ref[0, 0],
            None if allow is None else allow[0, 0], f"{wl.name} O f32")


@pytest.mark.parametrize("name", ["c3sq", "qb_sq"])
def test_smooth_q_full_size(name):
    wl = named(name)
    note(f"full size {wl}")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    o32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True,
                         smooth_q=True)
    torch.cuda.synchronize()
    N = wl.N
    rng = np.random.default_rng(wl.seed + 5)
    rows = np.array(sorted({0, 1, 127, 128, N // 2, N - 1} |
                           set(int(x) for x in rng.integers(0, N, 20))))
    for (b, h) in [(0, 0), (wl.B - 1, wl.H - 1)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref, allow = oracle_o(wl, inp.qf[sl], inp.kf[sl], inp.vf[sl], rows=rows)
        compare(to_np(o32[b, h, torch.from_numpy(rows).cuda()]), ref[0, 0],
                None if allow is None else allow[0, 0], f"{name} (b={b},h={h}) O f32")


def test_smooth_q_closer_to_exact_on_shared_q_bias():
    # the qb_sq inputs: Q and K carry per-channel biases ~ N(0, 4^2) shared by
    # all tokens; smoothing Q as well as K brings O closer to exact attention
    wl = named("qb_sq")
    inp = make_inputs(wl)
    q, k, v = inp.torch_tensors("cuda")
    rows = np.array(sorted(set(int(x) for x in np.random.default_rng(3).integers(0, wl.N, 48))))
    ri = torch.from_numpy(rows).cuda()
    o_sq = to_np(qa().sage_attn(q, k, v, pv_mode="fp16", out_f32=True, smooth_q=True)[:, :, ri])
    o_pl = to_np(qa().sage_attn(q, k, v, pv_mode="fp16", out_f32=True)[:, :, ri])
    ref = to_np(qa().ref_rows(q, k, v, ri))
    e_sq, e_pl = oracle.rel_l1(o_sq, ref), oracle.rel_l1(o_pl, ref)
    c_sq, c_pl = oracle.cos_sim(o_sq, ref), oracle.cos_sim(o_pl, ref)
    note(f"qb: smoothed Q RelL1 {e_sq:.5f} cos {c_sq:.7f} | K only RelL1 {e_pl:.5f} cos {c_pl:.7f}")
    assert e_sq < 0.95 * e_pl and c_sq > c_pl
