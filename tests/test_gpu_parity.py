"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Bar (each check names it):
* bit-exact: K column mean, delta_Q, delta_K, Q^, K^ (integer codes), fp16 V',
  E4M3 V^ codes and delta_V -- all decided in float32 on both sides;
* bit-exact: INT32 S = Q^ K^T from the attention kernel's MFMA code, on the
  oracle's own codes;
* O (float32 output of the same kernels): max |O - O_oracle| <= 2e-3 and
  cosine >= 0.9999; O in the 16-bit input dtype additionally within one ulp
  of that dtype (the final rounding).  FP8 and INT8 P~V: each element may
  exceed 2e-3 by the oracle's bound for 448 P~ (127 P~) values that lie, to
  float32 accuracy, on a rounding boundary of E4M3 (of the integers) (reading
  C-s; the count is reported).
Small cases compare every element; the five full workloads compare the whole
prepass and sampled query rows of O (first, last, ragged tail, diagonal and
seeded rows of several heads), computed by the oracle row by row.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import WORKLOADS, make_inputs, named, small

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-3
O_COS = 0.9999


def note(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def qa():
    import quantized_attention_qk_amd as m
    return m


def to_np(t):
    return t.detach().cpu().numpy()


def gpu_inputs(inp):
    return inp.torch_tensors("cuda")


# ---------------------------------------------------------------------------
SMALL = [
    small("s1", N=1, d=64), small("s63", N=63, d=128, causal=True),
    # FP16 P~V at d = 128, non-causal, runs 256-row workgroups of 8
    # wavefronts: one row, and one row past the first delta_Q block
    small("s1w", N=1, d=128), small("s129", N=129, d=128, dtype="bf16"),
    small("s65", N=65, d=64, dtype="bf16"), small("s197", N=197, d=64, pv_mode="fp8"),
    small("s300c", N=300, d=128, causal=True, dtype="bf16", pv_mode="fp8"),
    small("s1105", N=1105, d=64, H=1, causal=True, extras="kchan20"),
    small("s640", B=2, H=3, N=640, d=128, dtype="bf16", extras="q8_kbias5"),
    small("s257", N=257, d=128, pv_mode="fp8", extras="none"),
    # longer than the one-workgroup-per-head prepass handles: the multi-kernel
    # prepass, with ragged chunk, block and tile tails
    small("s2113", B=1, H=2, N=2113, d=64, pv_mode="fp8", extras="kbias4"),
    small("s2177", B=1, H=1, N=2177, d=128, dtype="bf16", causal=True),
    # scores that climb along the keys (recipe "ramp"): later tiles lie far
    # above the running maximum, so the FP16 kernel's steady-state steps take
    # their recompute branch (on a large share of the steps) and FP8 rescales
    # often
    small("r1000", N=1000, d=64, extras="ramp"),
    small("r2000b", N=2000, d=128, dtype="bf16", extras="ramp"),
    small("r1500c", N=1500, d=128, causal=True, extras="ramp"),
    small("r1000f8", N=1000, d=64, pv_mode="fp8", extras="ramp"),
    # INT8 P~V (all-INT8 variant): both d, causal, bf16, several heads, the
    # multi-kernel prepass and rising scores
    small("i197", N=197, d=64, pv_mode="int8"),
    small("i300c", N=300, d=128, causal=True, dtype="bf16", pv_mode="int8"),
    small("i640", B=2, H=3, N=640, d=128, dtype="bf16", pv_mode="int8", extras="q8_kbias5"),
    small("i2113", B=1, H=2, N=2113, d=128, pv_mode="int8", extras="kbias4"),
    small("i1105c", N=1105, d=64, H=1, causal=True, pv_mode="int8", extras="kchan20"),
    small("r1000i8", N=1000, d=64, pv_mode="int8", extras="ramp"),
    small("i1", N=1, d=128, pv_mode="int8"), small("i65c", N=65, d=64, causal=True,
                                                   pv_mode="int8", dtype="bf16"),
    # the two sides of the one-launch prepass limit (2048 tokens)
    small("b2048f8", N=2048, d=128, pv_mode="fp8", extras="kbias4"),
    small("b2049ci8", N=2049, d=64, causal=True, dtype="bf16", pv_mode="int8",
          extras="kchan20"),
]


def check_prepass(inp, res, vt, vs, heads=None):
    wl = inp.wl
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    qf, kf, vf = inp.qf, inp.kf, inp.vf
    if heads is not None:
        sel = (slice(None), heads)
        qf, kf, vf = qf[:, heads], kf[:, heads], vf[:, heads]
    pq = oracle.smooth_quant_qk(qf, kf)
    g = {k: to_np(t) for k, t in res.items()}
    if heads is not None:
        g = {k: v[:, heads] for k, v in g.items()}
    np.testing.assert_array_equal(g["k_mean"].view(np.uint32), pq["k_mean"].view(np.uint32),
                                  err_msg="k_mean bits")
    np.testing.assert_array_equal(g["q_scale"].view(np.uint32), pq["q_scale"].view(np.uint32),
                                  err_msg="q_scale bits")
    np.testing.assert_array_equal(g["k_scale"].view(np.uint32), pq["k_scale"].view(np.uint32),
                                  err_msg="k_scale bits")
    np.testing.assert_array_equal(g["q_i8"], pq["q_i8"], err_msg="q_i8")
    np.testing.assert_array_equal(g["k_i8"], pq["k_i8"], err_msg="k_i8")
    vv = qa().untile_v(vt, B, H, N, d, wl.pv_mode)
    if heads is not None:
        vv = vv[:, heads]
    _, codes, vscale = oracle.prep_v(vf, wl.pv_mode)
    if wl.pv_mode == "fp16":
        np.testing.assert_array_equal(vv.view(np.uint16), codes.view(np.uint16), err_msg="V' fp16")
    else:
        gs = to_np(vs) if heads is None else to_np(vs)[:, heads]
        np.testing.assert_array_equal(gs.view(np.uint32), vscale.view(np.uint32),
                                      err_msg="delta_V bits")
        np.testing.assert_array_equal(vv, codes, err_msg=f"V^ {wl.pv_mode} codes")
    return pq


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_prepass_bit_exact_small(wl):
    note(f"prepass {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    res = qa().smooth_quant_qk(q, k)
    vt, vs = qa().quant_v(v, wl.pv_mode)
    torch.cuda.synchronize()
    check_prepass(inp, res, vt, vs)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_debug_s_bit_exact(wl):
    note(f"debug S {wl}")
    inp = make_inputs(wl)
    pq = oracle.smooth_quant_qk(inp.qf, inp.kf)
    qi = torch.from_numpy(pq["q_i8"]).cuda()
    ki = torch.from_numpy(pq["k_i8"]).cuda()
    N = wl.N
    n32 = -(-N // 32) * 32
    for b in range(wl.B):
        for h in range(wl.H):
            s = to_np(qa().debug_s_i32(qi, ki, b, h, 0, n32, 0, n32))
            ref = np.zeros((n32, n32), np.int32)
            ref[:N, :N] = oracle.s_int32_tile(pq["q_i8"], pq["k_i8"], b, h, 0, N, 0, N)
            np.testing.assert_array_equal(s, ref, err_msg=f"S_i32 b={b} h={h}")


def compare_o(o_gpu, o_ref, what, allow=None):
    """max |O - O_oracle| <= 2e-3 and cosine >= 0.9999.  FP8 and INT8 P~V:
    `allow` is the oracle's per-element bound on O's move from P~ / delta_P
    values that lie, to float32 accuracy, on a rounding boundary of P^'s codes
    (reading C-s); the elements that need it are reported."""
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    cos = oracle.cos_sim(o_gpu, o_ref)
    extra = ""
    if allow is not None:
        over = err > O_MAX_ABS
        extra = f"  beyond 2e-3 (P^ boundary cases): {int(over.sum())}"
        assert np.all(err <= O_MAX_ABS + allow), \
            f"{what}: max excess {float((err - O_MAX_ABS - allow).max())}"
    note(f"{what}: max|dO| = {err.max():.3e}  cos = {cos:.7f}{extra}")
    if allow is None:
        assert err.max() <= O_MAX_ABS, f"{what}: max abs err {err.max()}"
    assert cos >= O_COS, f"{what}: cos {cos}"
    return err.max()


def oracle_o(wl, qf, kf, vf, **kw):
    """The oracle's O and, with a quantised P~ (FP8 or INT8 P~V), its bound on
    the effect of rounding-boundary cases of P^ (else None)."""
    if wl.pv_mode in ("fp8", "int8"):
        return oracle.sage_attention(qf, kf, vf, causal=wl.causal, pv_mode=wl.pv_mode,
                                     p_flip=True, **kw)
    return oracle.sage_attention(qf, kf, vf, causal=wl.causal, pv_mode=wl.pv_mode, **kw), None


def ulp16(x, dtype):
    x = np.abs(x)
    if dtype == "fp16":
        e = np.floor(np.log2(np.maximum(x, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_fwd_parity_small(wl):
    note(f"fwd {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    o32 = to_np(qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True))
    o16 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode)
    o16 = to_np(o16.float())
    ref, allow = oracle_o(wl, inp.qf, inp.kf, inp.vf)
    compare_o(o32, ref, f"{wl.name} O f32", allow)
    err16 = np.abs(o16 - ref)
    lim16 = O_MAX_ABS + ulp16(ref, wl.dtype) + (0.0 if allow is None else allow)
    assert np.all(err16 <= lim16), f"{wl.name} O 16-bit"


@pytest.mark.parametrize("wl", SMALL[:4], ids=lambda w: w.name)
def test_fwd_deterministic_and_guard_bands(wl):
    note(f"determinism {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    n = B * H * N * d
    pad = 4096
    buf = torch.full((n + 2 * pad,), 12345.0, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n].view(B, H, N, d)
    ws = torch.full((qa().workspace_bytes(B, H, N, d, wl.pv_mode) + 2 * pad,), 0xA5,
                    dtype=torch.uint8, device="cuda")
    wsv = ws[pad:pad + ws.numel() - 2 * pad]
    runs = []
    for _ in range(5):
        qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out=out, workspace=wsv,
                       out_f32=True)
        runs.append(out.clone())
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r.view(torch.int32), runs[0].view(torch.int32)), "not bitwise stable"
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + n:] == 12345.0)
    assert torch.all(ws[:pad] == 0xA5) and torch.all(ws[-pad:] == 0xA5)


@pytest.mark.parametrize("wl", [w for w in SMALL if w.name in ("s63", "s300c", "i300c", "i2113",
                                                                "s2177")],
                         ids=lambda w: w.name)
def test_stages_equal_whole_pass(wl):
    # sage_smooth_quant_qk + sage_quant_v + sage_attn_fwd_quantized on the
    # prepared operands give the whole pass's output bit for bit
    note(f"stages {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    whole = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    qk = qa().smooth_quant_qk(q, k)
    vp, vs = qa().quant_v(v, wl.pv_mode)
    staged = qa().sage_attn_quantized(qk, vp, vs, causal=wl.causal, pv_mode=wl.pv_mode,
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(staged.view(torch.int32), whole.view(torch.int32))


# ---------------------------------------------------------------------------
# The five full workloads, at their real sizes and in the launch configuration
# the benchmark times.
def sample_rows(N, causal, seed):
    """Edge rows, 24 seeded rows, and every row of one seeded 256-row span
    (aligned, so all 32 lanes of all eight wavefronts of one workgroup, or of
    two 128-row workgroups)."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, 63, 64, 127, 128, N - 1, N - 2, N // 2, (N // 128) * 128 - 1}
    rows |= set(int(x) for x in rng.integers(0, N, 24))
    span = 256 * int(rng.integers(0, max(1, N // 256)))
    rows |= set(range(span, span + 256))
    return np.array(sorted(r for r in rows if 0 <= r < N))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5", "c3i8", "c4i8", "c3_shard8"])
def test_full_workload(name):
    wl = named(name)
    note(f"full workload {name}: {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    B, H, N, d = wl.B, wl.H, wl.N, wl.d
    # prepass over the whole tensors (bit-exact), a subset of heads for time
    res = qa().smooth_quant_qk(q, k)
    vt, vs = qa().quant_v(v, wl.pv_mode)
    torch.cuda.synchronize()
    rng = np.random.default_rng(wl.seed + 100)
    heads_h = sorted(set([0, H - 1] + [int(x) for x in rng.integers(0, H, 2)]))
    note(f"{name}: prepass check on heads {heads_h}")
    check_prepass(inp, res, vt, vs, heads=heads_h)
    del res, vt, vs
    # forward in the benchmark's configuration, O in float32 and 16-bit
    o32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    o16 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode)
    torch.cuda.synchronize()
    rows = sample_rows(N, wl.causal, wl.seed)
    pairs = sorted(set([(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H)))
                                                  for _ in range(2)]))
    for (b, h) in pairs:
        note(f"{name}: rows of head (b={b}, h={h})")
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref, allow = oracle_o(wl, inp.qf[sl], inp.kf[sl], inp.vf[sl], rows=rows)
        ref = ref[0, 0]
        allow = None if allow is None else allow[0, 0]
        g32 = to_np(o32[b, h, torch.from_numpy(rows).cuda()])
        g16 = to_np(o16[b, h, torch.from_numpy(rows).cuda()].float())
        # the five workloads meet 2e-3 with no allowance for P^ boundary
        # cases; the allowance stays for the INT8 P~V variants of c3, c4
        strict = name in ("c1", "c2", "c3", "c4", "c5", "c3_shard8")
        compare_o(g32, ref, f"{name} (b={b},h={h}) O f32", None if strict else allow)
        lim16 = O_MAX_ABS + ulp16(ref, wl.dtype) + (0.0 if allow is None else allow)
        assert np.all(np.abs(g16 - ref) <= lim16), "16-bit O"


@pytest.mark.parametrize("name", ["t7_cogvideox", "t7_unidiffuser", "t7_ultrapixel", "t7_llama2",
                                  "t7_timm"])
def test_table7_shapes(name):
    # real-model shapes (B, H, N, d) of the pages' Table 7, full size, with
    # ragged token counts 17776, 1105 and 197: sampled rows of two heads
    from workloads import TABLE7
    wl = TABLE7[name]
    note(f"table-7 shape {name}: {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    B, H, N = wl.B, wl.H, wl.N
    o32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    torch.cuda.synchronize()
    rows = sample_rows(N, wl.causal, wl.seed)
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.sage_attention(inp.qf[sl], inp.kf[sl], inp.vf[sl], causal=wl.causal,
                                    pv_mode=wl.pv_mode, rows=rows)[0, 0]
        compare_o(to_np(o32[b, h, torch.from_numpy(rows).cuda()]), ref,
                  f"{name} (b={b},h={h}) O f32")


# ---------------------------------------------------------------------------
# INT8 P~V keeps O as an INT32 sum of the tiles' P^ V^ for heads of up to 2^17
# keys and converts each tile's product to float beyond.  Q = 0 makes every
# score equal, so every P^ is 127; V constant per channel makes every V^ +-127.
# At 2^17 keys each INT32 sum is then +-2^17 127^2 = +-2114060288, the bound
# the kernel relies on, and O must be V itself (closed form).
@pytest.mark.parametrize("N,d,causal", [(1 << 17, 128, False), (1 << 17, 64, True),
                                        ((1 << 17) + 1, 128, False)],
                         ids=["acc_bound_d128", "acc_bound_d64c", "above_bound_d128"])
def test_int8_accumulator_bound(N, d, causal):
    note(f"int8 accumulator bound N={N} d={d} causal={causal}")
    g = torch.Generator().manual_seed(N + d)
    q = torch.zeros(1, 1, N, d, dtype=torch.float16)
    k = torch.randn(1, 1, N, d, generator=g).to(torch.float16)
    col = (torch.rand(d, generator=g) * 4 + 0.5) * torch.where(torch.arange(d) % 2 == 0, 1.0, -1.0)
    v = col.to(torch.float16).expand(1, 1, N, d).contiguous()
    o = qa().sage_attn(q.cuda(), k.cuda(), v.cuda(), causal=causal, pv_mode="int8", out_f32=True)
    torch.cuda.synchronize()
    ref = col.to(torch.float16).double().numpy()
    err = np.abs(to_np(o)[0, 0] - ref[None, :])
    note(f"  max |O - V| = {err.max():.3e}")
    # INT32 sums: only the final conversions and the float32 row sum round.
    # Beyond 2^17 keys each of the N/64 tile products is added to a float32 O
    # of up to 2^31 units, each addition rounding by half an ulp (2^-24 rel).
    rel = 1e-5 if N <= (1 << 17) else 1e-5 + (N / 64) * 2.0 ** -24
    assert err.max() <= rel * np.abs(ref).max()


# ---------------------------------------------------------------------------
# Maximum sizes: one head of about a million tokens (K^ tile index up to
# 16384, a V' head of 256 MiB), ragged, in both P~V modes.
@pytest.mark.parametrize("wl", [
    small("long1m", B=1, H=1, N=(1 << 20) + 37, d=128, dtype="bf16", pv_mode="fp16", seed=31),
    small("long512kc8", B=1, H=1, N=(1 << 19) + 5, d=64, causal=True, pv_mode="fp8", seed=32),
    small("long512kci8", B=1, H=1, N=(1 << 19) + 3, d=128, causal=True, pv_mode="int8",
          seed=33),
], ids=lambda w: w.name)
def test_long_sequence(wl):
    note(f"long sequence {wl}")
    inp = make_inputs(wl)
    q, k, v = gpu_inputs(inp)
    res = qa().smooth_quant_qk(q, k)
    vt, vs = qa().quant_v(v, wl.pv_mode)
    torch.cuda.synchronize()
    check_prepass(inp, res, vt, vs)
    del res, vt, vs
    o32 = qa().sage_attn(q, k, v, causal=wl.causal, pv_mode=wl.pv_mode, out_f32=True)
    torch.cuda.synchronize()
    N = wl.N
    rows = np.array(sorted({0, 1, 63, 64, 12345, N // 2, N - 65, N - 2, N - 1}))
    ref, allow = oracle_o(wl, inp.qf, inp.kf, inp.vf, rows=rows)
    g32 = to_np(o32[0, 0, torch.from_numpy(rows).cuda()])
    compare_o(g32, ref[0, 0], f"{wl.name} O f32", None if allow is None else allow[0, 0])
