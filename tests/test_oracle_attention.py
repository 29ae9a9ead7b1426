"""Pins for the oracle's tiled online-softmax attention.

* With the identity quantiser the tiled algorithm ("SageAttention ..." detail
  page, §3 Algorithm 1) must reproduce textbook softmax attention (§4 symbol
  table: S = QK^T/sqrt(d), P = softmax(S), O = PV), computed in one shot.
* Smoothing is exact under softmax (§4 Eq. 6 and the shift-invariance argument
  after it): smoothed and unsmoothed full-precision outputs agree.
* max P~ = 1 in every row (§2 assumptions; §7 static P~ scale).
* When quantisation is lossless by construction, the INT8 path equals the
  textbook result exactly (pins the block scales and 1/sqrt(d)).
* FP8 P~V (SageAttention2++ review page, section 三): the output stays within
  the error bound implied by E4M3 rounding of P^ = 448 P~ and of V.
* INT8 P~V (the all-INT8 variant of the detail page, §3 Figure 5, with the
  static delta_P = 1/127 of §7): equal scores average the INT8 V exactly, a
  dominant key returns its V row, and the rounding of P^ = 127 P~ moves O by
  at most half a step per key.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (KV_TILE, brute_attention, cos_sim, prep_v, rel_l1,
                    sage_attention, smooth_quant_qk)
from oracle.codecs import e4m3_decode, fp16_round
from workloads import make_inputs, small

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))

# Table 7 of the SageAttention detail page lists token counts 197 and 1105;
# they serve here as ragged-tail cases next to tile-boundary sizes.
N_CASES = [1, 63, 64, 65, 129, 197, 300]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", N_CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_identity_quantizer_equals_textbook(d, N, causal):
    inp = make_inputs(small(N=N, d=d, seed=N + d, extras="kbias4"))
    o = sage_attention(inp.qf, inp.kf, inp.vf, causal=causal, pv_mode="none", quant="none",
                       smooth=False)
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=causal)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identity_quantizer_1105_tokens(causal):
    inp = make_inputs(small(N=1105, d=64, H=1, seed=1105))
    o = sage_attention(inp.qf, inp.kf, inp.vf, causal=causal, pv_mode="none", quant="none")
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=causal)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("extras", ["kbias4", "kchan20"])
def test_smoothing_is_exact_in_full_precision(causal, extras):
    inp = make_inputs(small(N=333, d=128, seed=21, extras=extras))
    on = sage_attention(inp.qf, inp.kf, inp.vf, causal=causal, pv_mode="none", quant="none",
                        smooth=True)
    off = sage_attention(inp.qf, inp.kf, inp.vf, causal=causal, pv_mode="none", quant="none",
                         smooth=False)
    assert np.abs(on - off).max() <= 1e-6


def test_hand_worked_two_tokens():
    # d = 4, q = [2 ln 3, 0, 0, 0] for both rows, k0 = 0, k1 = e_0:
    # scores [0, ln 3] -> weights [1/4, 3/4]; causal row 0 sees only key 0.
    q = np.zeros((1, 1, 2, 4), np.float32)
    k = np.zeros((1, 1, 2, 4), np.float32)
    v = np.zeros((1, 1, 2, 4), np.float32)
    q[0, 0, :, 0] = 2 * math.log(3.0)
    k[0, 0, 1, 0] = 1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 0, 1, 1] = 1.0
    nc = sage_attention(q, k, v, causal=False, pv_mode="none", quant="none")
    c = sage_attention(q, k, v, causal=True, pv_mode="none", quant="none")
    np.testing.assert_allclose(nc[0, 0], [[0.25, 0.75, 0, 0]] * 2, atol=1e-6)
    np.testing.assert_allclose(c[0, 0], [[1, 0, 0, 0], [0.25, 0.75, 0, 0]], atol=1e-6)


def test_hand_worked_int8_fp16():
    # The quantised example of test_oracle_quant.test_smooth_quant_hand_worked:
    # row 0 scores S = 127*(+-127) * delta_Q * delta_K with the float32 scales
    # delta_Q = fp32(2/127), delta_K = fp32(1/127), i.e. +-2 up to their rounding
    # -> P~ = [exp(-2 s0), 1], l = 1 + exp(-2 s0), P~ rounded to fp16 before P~V.
    q = np.zeros((1, 1, 2, 4), np.float32)
    k = np.zeros((1, 1, 2, 4), np.float32)
    q[0, 0, :, 0] = [4.0, 2.0]
    k[0, 0, :, 0] = [1.0, 3.0]
    v = np.arange(1, 9, dtype=np.float32).reshape(1, 1, 2, 4)
    o = sage_attention(q, k, v, causal=False, pv_mode="fp16")
    v64 = v.astype(np.float64)
    dq = float(np.float32(2) / np.float32(127))
    dk = float(np.float32(1) / np.float32(127))
    for row, code in ((0, 127), (1, 64)):      # row 1: 63.5 ties to even -> 64
        s = code * 127 * dq * dk
        p = float(np.float16(math.exp(-2 * s)))      # e.g. row 0: fp16(e^-4) = 0.0183105...
        expect = (p * v64[0, 0, 0] + v64[0, 0, 1]) / (1.0 + math.exp(-2 * s))
        np.testing.assert_allclose(o[0, 0, row], expect, rtol=1e-12)


def test_hand_worked_fp8_static_scale():
    # Two keys with scores [0, s], 448 e^s = 17.2: P^ = E4M3(448 P~) = [448, 18]
    # (17.2 lies above the 16/18 midpoint), so with V unquantised
    # O = (448 v0 + 18 v1) / (448 (1 + e^s)).  A wrong static scale moves P^.
    s = math.log(17.2 / 448.0)
    q = np.zeros((1, 1, 2, 4), np.float32)
    k = np.zeros((1, 1, 2, 4), np.float32)
    q[0, 0, 1, 0] = 2 * s                        # d = 4: S = q.k / 2
    k[0, 0, 1, 0] = 1.0
    v = np.arange(1, 9, dtype=np.float32).reshape(1, 1, 2, 4)
    o = sage_attention(q, k, v, causal=False, pv_mode="fp8", quant="none", smooth=False)
    s32 = float(np.float32(2 * s)) / 2
    v64 = v.astype(np.float64)
    expect = (448 * v64[0, 0, 0] + 18 * v64[0, 0, 1]) / (448 * (1 + math.exp(s32)))
    np.testing.assert_allclose(o[0, 0, 1], expect, rtol=1e-12)
    np.testing.assert_allclose(o[0, 0, 0], (v64[0, 0, 0] + v64[0, 0, 1]) / 2, rtol=1e-12)


@pytest.mark.parametrize("pv_mode", ["fp16", "fp8"])
@pytest.mark.parametrize("causal", [False, True])
def test_ptilde_in_unit_interval_and_max_one(pv_mode, causal):
    inp = make_inputs(small(N=450, d=64, seed=31, causal=causal))
    _, recs = sage_attention(inp.qf, inp.kf, inp.vf, causal=causal, pv_mode=pv_mode,
                             record=True)
    for rec in recs.values():
        pm = rec["pmax_tiles"]
        assert np.all(pm <= 1.0) and np.all(pm >= 0.0)
        assert np.all(pm.max(axis=1) == 1.0)        # exp(0) in the block of the final max
        assert np.all(rec["l"] >= 1.0)


def _exact_int8_case(d=64, N=200, seed=0):
    """Inputs whose INT8 quantisation is lossless: Q/sqrt(d) and K - mean are
    integers times a per-block power of two, each block holding a +-127.
    Every 64-token K block is made of a half and its negation, so the column
    mean is exactly 0 (and the float32 sums are exact)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(N, d)).astype(np.float64)
    for j in range(0, N, 128):
        q[j, 0] = 127
        q[j:j + 128] *= 2.0 ** ((j // 128) % 3 - 1)
    k = np.zeros((N, d))
    for j in range(0, N, 64):
        n = min(64, N - j)
        h = n // 2
        if h == 0:
            continue
        blk = rng.integers(-127, 128, size=(h, d)).astype(np.float64)
        blk[0, 1] = 127
        s = 2.0 ** ((j // 64) % 4 - 2)
        k[j:j + h] = blk * s
        k[j + h:j + 2 * h] = -blk * s
    qf = (q * np.sqrt(d)).astype(np.float32)[None, None]   # Q/sqrt(d) = q exactly (d = 64)
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    return qf, k.astype(np.float32)[None, None], v


@pytest.mark.parametrize("causal", [False, True])
def test_int8_path_exact_when_quantisation_lossless(causal):
    qf, kf, vf = _exact_int8_case(N=200 if causal else 333)
    pq = smooth_quant_qk(qf, kf)
    assert np.all(pq["k_mean"] == 0)
    o = sage_attention(qf, kf, vf, causal=causal, pv_mode="none", prep=pq)
    ref = brute_attention(qf, kf, vf, causal=causal)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_fp16_pv_rounding_bound():
    inp = make_inputs(small(N=500, d=64, seed=41))
    o16 = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp16")
    o = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none")
    diff = np.abs(o16 - o)
    # P~ and V rounded to fp16: relative error <= 2^-11 each
    bound = 2 * 2.0 ** -11 * np.abs(inp.vf).max() + 1e-12
    assert diff.max() <= bound
    assert diff.max() > 0         # the rounding is applied


def test_fp8_pv_error_bound():
    inp = make_inputs(small(N=500, d=64, seed=42))
    o8 = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp8")
    o = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none")
    # relative error of each P^ V^ product term <= (1 + 2^-4)^2 - 1 for normal
    # codes; subnormal P^ (448 P~ < 2^-6) adds at most 2^-10/448 per key.
    vmax = np.abs(inp.vf).max()
    N = inp.vf.shape[2]
    _, recs = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none", record=True)
    l = np.stack([recs[(0, h)]["l"] for h in range(inp.vf.shape[1])])[None]     # [1, H, N]
    bound = (((1 + 2.0 ** -4) ** 2 - 1) * vmax + N * 2.0 ** -10 / 448 * vmax / l[..., None]
             + 2.0 ** -10 * vmax / 448 * (1 + 2.0 ** -4))
    assert np.all(np.abs(o8 - o) <= bound + 1e-12)


def test_accuracy_levels_near_table2():
    # Advisory: [SA] §5 Table 2 reports CosSim 99.99% (INT8 + FP16) and
    # 99.94% (INT8 + E4M3) on real layers; synthetic data must land close.
    inp = make_inputs(small(N=1024, d=64, H=2, seed=0, extras="kbias4"))
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=False)
    o16 = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp16")
    o8 = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp8")
    assert cos_sim(o16, ref) >= GOLD["table2_int8_fp16"]["cos"] - 2e-4
    assert cos_sim(o8, ref) >= GOLD["table2_int8_e4m3"]["cos"] - 1e-3
    assert rel_l1(o16, ref) < rel_l1(o8, ref)


def test_smoothing_improves_int8_accuracy():
    # direction of [SA] §5 Table 1: per-block INT8 with smooth K beats without
    inp = make_inputs(small(N=1024, d=64, H=2, seed=0, extras="kbias4"))
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=False)
    on = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp16", smooth=True)
    off = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="fp16", smooth=False)
    assert rel_l1(on, ref) < 0.5 * rel_l1(off, ref)
    assert cos_sim(on, ref) > cos_sim(off, ref)


def test_rows_subset_matches_full_and_causality():
    inp = make_inputs(small(N=260, d=64, seed=51, causal=True))
    full = sage_attention(inp.qf, inp.kf, inp.vf, causal=True, pv_mode="fp8")
    rows = np.array([0, 1, 63, 64, 127, 128, 200, 259])
    sub = sage_attention(inp.qf, inp.kf, inp.vf, causal=True, pv_mode="fp8", rows=rows)
    np.testing.assert_allclose(sub, full[:, :, rows], rtol=0, atol=1e-12)
    # in full precision, row i ignores keys and values after i
    k2, v2 = inp.kf.copy(), inp.vf.copy()
    k2[:, :, 101:] += 3.0
    v2[:, :, 101:] -= 5.0
    a = sage_attention(inp.qf, inp.kf, inp.vf, causal=True, pv_mode="none", quant="none",
                       smooth=False)
    b = sage_attention(inp.qf, k2, v2, causal=True, pv_mode="none", quant="none", smooth=False)
    np.testing.assert_array_equal(a[:, :, :101], b[:, :, :101])
    assert not np.allclose(a[:, :, 101:], b[:, :, 101:])


def test_kv_tile_contract():
    assert KV_TILE == 64


def test_fp8_flip_bound_covers_perturbed_rounding():
    """The FP8 boundary bound of the oracle (reading C-s): when every 448 P~ is
    perturbed by a relative amount below the band, codes that flip lie within
    the band, so O moves by at most the returned bound; with a band wide enough
    to flip codes, O does move (the bound is not vacuous)."""
    import oracle
    import oracle.sage_oracle as so
    from oracle.codecs import e4m3_decode, e4m3_encode
    from workloads import small, make_inputs
    wl = small("flip", N=150, d=64, pv_mode="fp8", extras="ramp")
    inp = make_inputs(wl)
    pq = oracle.smooth_quant_qk(inp.qf, inp.kf)
    _, codes, vscale = oracle.prep_v(inp.vf, "fp8")
    vvals = e4m3_decode(codes)
    b, h = 0, 1
    args = (pq["q_i8"][b, h].astype(np.float64), pq["q_scale"][b, h, np.arange(wl.N) // 128],
            pq["k_i8"][b, h].astype(np.float64), pq["k_scale"][b, h, np.arange(wl.N) // 64],
            vvals[b, h], vscale[b, h].astype(np.float64))
    band = 2e-3
    o, bound = so.attention(*args, causal=False, p_round=so._p_round_for("fp8"), p_flip=band)
    moved = 0.0
    for rho in (0.999 * band, -0.999 * band):
        pr = lambda p, r=rho: e4m3_decode(e4m3_encode(p * 448.0 * (1.0 + r))) / 448.0
        o2 = so.attention(*args, causal=False, p_round=pr)
        d = np.abs(o2 - o)
        assert np.all(d <= bound + 1e-12), float((d - bound).max())
        moved = max(moved, float(d.max()))
    assert moved > 0.0


def test_fp8_codes_follow_the_exact_max():
    """Why FP8 P~V keeps the exact running max.  P^ = E4M3(448 P~) has 3
    mantissa bits, so scaling every 448 P~ by a common factor 1 + r (O and l
    alike, as a max rounded up onto a grid would) moves codes across rounding
    boundaries: at r = -1e-4 (a max 1.4e-4 log2 units high) O moves by more
    than the 2e-3 parity bar on these inputs, although without rounding the
    factor would cancel in O / l exactly.  A shift of 1e-6 (float32 rounding
    of the argument) stays far inside it."""
    import oracle.sage_oracle as so
    from oracle.codecs import e4m3_encode
    wl = small("s197", N=197, d=64, pv_mode="fp8", seed=11, extras="kbias4")
    inp = make_inputs(wl)
    pq = smooth_quant_qk(inp.qf, inp.kf)
    _, codes, vscale = prep_v(inp.vf, "fp8")
    vvals = e4m3_decode(codes)
    N = wl.N
    args = (pq["q_i8"][0, 0].astype(np.float64), pq["q_scale"][0, 0, np.arange(N) // 128],
            pq["k_i8"][0, 0].astype(np.float64), pq["k_scale"][0, 0, np.arange(N) // 64],
            vvals[0, 0], vscale[0, 0].astype(np.float64))
    o = so.attention(*args, causal=False, p_round=so._p_round_for("fp8"))
    moved = {}
    for r in (-1e-4, 1e-6):
        pr = lambda p, r=r: e4m3_decode(e4m3_encode(p * 448.0 * (1.0 + r))) / (448.0 * (1.0 + r))
        moved[r] = float(np.abs(so.attention(*args, causal=False, p_round=pr) - o).max())
    assert moved[-1e-4] > 2e-3, moved
    assert moved[1e-6] < 1e-5, moved


def _int8_head_args(qf, kf, vf, b=0, h=0):
    import oracle
    N = qf.shape[2]
    pq = oracle.smooth_quant_qk(qf, kf)
    vals, _, vscale = oracle.prep_v(vf, "int8")
    return (pq["q_i8"][b, h].astype(np.float64), pq["q_scale"][b, h, np.arange(N) // 128],
            pq["k_i8"][b, h].astype(np.float64), pq["k_scale"][b, h, np.arange(N) // 64],
            vals[b, h], vscale[b, h].astype(np.float64))


@pytest.mark.parametrize("causal", [False, True])
def test_int8_pv_equal_scores_average_v(causal):
    # Q = 0: every score is 0, every P~ = 1, every P^ = 127 (no rounding), so
    # row i of O is the mean of the dequantised INT8 V over its visible keys.
    inp = make_inputs(small(N=150, d=64, seed=61))
    qf = np.zeros_like(inp.qf)
    o = sage_attention(qf, inp.kf, inp.vf, causal=causal, pv_mode="int8")
    _, codes, vscale = prep_v(inp.vf, "int8")
    deq = codes.astype(np.float64) * vscale[:, :, None, :].astype(np.float64)
    if causal:
        ref = np.cumsum(deq, axis=2) / np.arange(1, 151)[None, None, :, None]
    else:
        ref = np.broadcast_to(deq.mean(axis=2, keepdims=True), deq.shape)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal,dom", [(False, 77), (True, 0)])
def test_int8_pv_dominant_key_returns_its_row(causal, dom):
    # One key scores 40 above every other (e^-40: P^ = 0 for the rest and l = 1
    # to float64 precision): O = the dequantised INT8 V row of that key.
    N, d = 130, 64
    rng = np.random.default_rng(62)
    qf = np.zeros((1, 1, N, d), np.float32)
    qf[..., 0] = 32.0                      # Q/sqrt(d) = 4 in channel 0
    kf = (0.01 * rng.standard_normal((1, 1, N, d))).astype(np.float32)
    kf[0, 0, dom, 0] += 10.0
    vf = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    o = sage_attention(qf, kf, vf, causal=causal, pv_mode="int8")
    _, codes, vscale = prep_v(vf, "int8")
    row = codes[0, 0, dom].astype(np.float64) * vscale[0, 0].astype(np.float64)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(row, (N, d)), rtol=0, atol=1e-13)


def test_int8_pv_rounding_bound():
    # |round(127 P~)/127 - P~| <= 1/254 for every key, and alpha <= 1, so O
    # moves from its exact-P~ value (same INT8 V) by at most
    # (1/254) sum_keys |V_deq| / l per element.
    import oracle.sage_oracle as so
    inp = make_inputs(small(N=300, d=64, seed=63, extras="kbias4"))
    args = _int8_head_args(inp.qf, inp.kf, inp.vf, 0, 1)
    oi = so.attention(*args, causal=False, p_round=so._p_round_for("int8"))
    oe, rec = so.attention(*args, causal=False, p_round=lambda p: p, record=True)
    vdeq = np.abs(args[4] * args[5][None, :])
    bound = vdeq.sum(axis=0)[None, :] / 254.0 / rec["l"][:, None]
    diff = np.abs(oi - oe)
    assert np.all(diff <= bound * (1 + 1e-12))
    assert diff.max() > 0
    # and the oracle's full pass uses exactly this per-head computation
    full = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="int8")
    np.testing.assert_allclose(full[0, 1], oi, rtol=0, atol=0)


def test_int8_flip_bound_covers_perturbed_rounding():
    """The INT8 counterpart of the FP8 boundary bound (reading C-s): every
    127 P~ perturbed by a relative amount below the band moves O by at most the
    returned bound, and a band this wide does move it."""
    import oracle.sage_oracle as so
    wl = small("flip8", N=150, d=64, pv_mode="int8", extras="ramp")
    inp = make_inputs(wl)
    args = _int8_head_args(inp.qf, inp.kf, inp.vf, 0, 1)
    band = 2e-3
    o, bound = so.attention(*args, causal=False, p_round=so._p_round_for("int8"), p_flip=band,
                            p_codec="int8")
    moved = 0.0
    for rho in (0.999 * band, -0.999 * band):
        pr = lambda p, r=rho: np.clip(np.rint(p * 127.0 * (1.0 + r)), 0, 127) / 127.0
        o2 = so.attention(*args, causal=False, p_round=pr)
        d = np.abs(o2 - o)
        assert np.all(d <= bound + 1e-12), float((d - bound).max())
        moved = max(moved, float(d.max()))
    assert moved > 0.0


def test_int8_pv_accuracy_levels_table2():
    """[SA] §5 Table 2 puts INT8 P~,V below E4M3 (cosine 99.70% vs 99.94% on
    real layers).  Its mechanism: with delta_P = 1/127 every P~ below 1/254
    becomes P^ = 0.  A sink row (one key 6 above a flat background, whose V
    has a nonzero mean) loses the whole background: O is the sink's INT8 V
    row over l, exactly, and the cosine falls below FP8's.  On diffuse
    synthetic rows (no such loss) INT8 V is finer than E4M3, and the level is
    at least the page's INT8 cosine."""
    N, d = 1024, 64
    rng = np.random.default_rng(5)
    qf = np.zeros((1, 1, N, d), np.float32)
    qf[..., 0] = 8.0                                   # Q/sqrt(d) = 1 in channel 0
    kf = (0.05 * rng.standard_normal((1, 1, N, d))).astype(np.float32)
    kf[0, 0, 0, 0] += 6.0
    vf = (rng.standard_normal((1, 1, N, d)) + 1.0).astype(np.float32)
    ref = brute_attention(qf, kf, vf, causal=False)
    o8 = sage_attention(qf, kf, vf, causal=False, pv_mode="fp8")
    _, recs = sage_attention(qf, kf, vf, causal=False, pv_mode="int8", record=True)
    oi = sage_attention(qf, kf, vf, causal=False, pv_mode="int8")
    _, codes, vscale = prep_v(vf, "int8")
    row = codes[0, 0, 0].astype(np.float64) * vscale[0, 0].astype(np.float64)
    np.testing.assert_allclose(oi[0, 0], row[None, :] / recs[(0, 0)]["l"][:, None], rtol=1e-13,
                               atol=0)
    assert cos_sim(oi, ref) < cos_sim(o8, ref) - 0.05
    inp = make_inputs(small(N=1024, d=64, H=2, seed=0, extras="kbias4"))
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=False)
    oi = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="int8")
    assert cos_sim(oi, ref) >= GOLD["table2_int8_int8"]["cos"]
