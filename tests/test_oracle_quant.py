"""Pins for the oracle's prepass: the K column mean, the INT8 block quantiser,
V preparation and the exact INT32 product.

Pages: "SageAttention: Accurate 8-Bit Attention ..." detail page, §3
Algorithm 1 and §4 Eq. 6 (smooth K: subtract the token mean of every channel);
"SageAttention2++ ..." review page, section 三 core formulas
(delta = max|X|/127, X^ = round(X/delta); delta_V = colmax|V|/448); the
all-INT8 variant's V (detail page §3 Figure 5) with delta_V = colmax|V|/127.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (K_BLOCK, Q_BLOCK, column_mean, inv_sqrt_d, prep_v,
                    quantize_int8_blocks, s_int32_tile, smooth_quant_qk)
from oracle.codecs import e4m3_decode
from workloads import make_inputs, small

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def f32_correctly_rounded(fr: Fraction) -> np.float32:
    """The float32 nearest to an exact rational (ties to even), found by
    comparing exact rationals of the neighbouring float32 candidates."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda f: (abs(Fraction(float(f)) - fr),
                                     int(np.array(f, np.float32).view(np.uint32)) & 1))
    return np.float32(best)


def test_mean_exact_on_integer_keys():
    # integer-valued K: every float32 partial sum is exact, so the mean must be
    # the correctly rounded float32 of the exact rational sum/N.
    rng = np.random.default_rng(1)
    for N in (1, 5, 255, 256, 257, 1000, 1105):
        k = rng.integers(-20, 21, size=(1, 2, N, 8)).astype(np.float32)
        m = column_mean(k)
        for h in range(2):
            for c in range(8):
                exact = Fraction(int(k[0, h, :, c].astype(np.int64).sum()), N)
                assert m[0, h, c] == f32_correctly_rounded(exact), (N, h, c)


def test_mean_error_bound_general():
    inp = make_inputs(small(N=3001, d=64, seed=3))
    m = column_mean(inp.kf).astype(np.float64)
    exact = inp.kf.astype(np.float64).mean(axis=2)
    N = inp.kf.shape[2]
    # sequential float32 summation of n terms: |err| <= (n-1) u sum|x|, u = 2^-24,
    # here n <= 256 per chunk plus ceil(N/256) partials, then one division.
    n_terms = 256 + (N + 255) // 256
    bound = n_terms * 2.0 ** -24 * np.abs(inp.kf.astype(np.float64)).sum(axis=2) / N
    bound += 2.0 ** -24 * np.abs(exact) + 1e-30
    assert np.all(np.abs(m - exact) <= bound)


def test_quantizer_hand_worked_block():
    # block [0.5, -1.0, 0.25, 2.0]: a = 2, r = 127/2 = 63.5,
    # x*r = [31.75, -63.5, 15.875, 127] -> RNE [32, -64, 16, 127], delta = 2/127
    x = np.array([0.5, -1.0, 0.25, 2.0], np.float32).reshape(1, 1, 1, 4)
    codes, delta = quantize_int8_blocks(x, Q_BLOCK)
    assert codes.ravel().tolist() == [32, -64, 16, 127]
    assert delta.ravel()[0] == np.float32(2.0) / np.float32(127.0)


@pytest.mark.parametrize("N,block", [(1, 128), (200, 128), (256, 128), (197, 64), (1105, 64)])
def test_quantizer_closed_forms(N, block):
    inp = make_inputs(small(N=N, d=64, seed=N))
    x = inp.qf * np.float32(3.0)
    codes, delta = quantize_int8_blocks(x, block)
    assert codes.dtype == np.int8
    assert codes.min() >= -GOLD["int8_range"]["value"] and codes.max() <= GOLD["int8_range"]["value"]
    B, H, _, d = x.shape
    nb = -(-N // block)
    assert delta.shape == (B, H, nb)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                xb = x[b, h, j * block:(j + 1) * block].astype(np.float64)
                cb = codes[b, h, j * block:(j + 1) * block].astype(np.float64)
                a = np.abs(xb).max()
                assert delta[b, h, j] == np.float32(np.float32(a) / np.float32(127.0))
                # the absmax element maps to +-127
                i = np.unravel_index(np.abs(xb).argmax(), xb.shape)
                assert abs(cb[i]) == 127 and np.sign(cb[i]) == np.sign(xb[i])
                # rounding to nearest: |x * 127/a - code| <= 1/2 (+ float32 product rounding)
                assert np.all(np.abs(xb * (127.0 / a) - cb) <= 0.5 + 127 * 2.0 ** -23)
                # dequantisation error <= delta/2 (+ scale rounding)
                assert np.all(np.abs(cb * delta[b, h, j] - xb) <= delta[b, h, j] * (0.5 + 1e-5))


def test_quantizer_zero_block():
    x = np.zeros((1, 1, 70, 4), np.float32)
    x[0, 0, 64:] = 1.0
    codes, delta = quantize_int8_blocks(x, 64)
    assert delta[0, 0, 0] == 0 and np.all(codes[0, 0, :64] == 0)
    assert delta[0, 0, 1] == np.float32(1.0) / np.float32(127.0) and np.all(codes[0, 0, 64:] == 127)


def test_smooth_quant_hand_worked():
    # N=2, d=4 (1/sqrt(d) = 0.5 exactly):
    # Q' = Q/2 = [[2],[1]] -> a = 2, r = 63.5 -> codes [127, 64 (63.5 ties to even)]
    # mean K = 2 -> K~ = [-1, 1] -> codes [-127, 127], delta_K = 1/127
    q = np.zeros((1, 1, 2, 4), np.float32)
    k = np.zeros((1, 1, 2, 4), np.float32)
    q[0, 0, :, 0] = [4.0, 2.0]
    k[0, 0, :, 0] = [1.0, 3.0]
    pq = smooth_quant_qk(q, k)
    assert pq["k_mean"][0, 0].tolist() == [2.0, 0.0, 0.0, 0.0]
    assert pq["q_i8"][0, 0, :, 0].tolist() == [127, 64]
    assert pq["k_i8"][0, 0, :, 0].tolist() == [-127, 127]
    assert pq["q_scale"][0, 0, 0] == np.float32(2.0) / np.float32(127.0)
    assert pq["k_scale"][0, 0, 0] == np.float32(1.0) / np.float32(127.0)


def test_smoothed_k_reconstructs_k():
    # K^ * delta_K + mean reproduces K within half a quantisation step; a sign
    # error in the smoothing or a wrong block index breaks this.
    inp = make_inputs(small(N=300, d=128, seed=4, extras="kbias4"))
    pq = smooth_quant_qk(inp.qf, inp.kf)
    N = inp.kf.shape[2]
    dk = pq["k_scale"][:, :, np.arange(N) // K_BLOCK][..., None].astype(np.float64)
    rec = pq["k_i8"].astype(np.float64) * dk + pq["k_mean"][:, :, None, :]
    assert np.all(np.abs(rec - inp.kf) <= dk * 0.5 * (1 + 1e-5) + 1e-6)
    dq = pq["q_scale"][:, :, np.arange(N) // Q_BLOCK][..., None].astype(np.float64)
    recq = pq["q_i8"].astype(np.float64) * dq / float(inv_sqrt_d(128))
    assert np.all(np.abs(recq - inp.qf) <= dq * 0.5 * (1 + 1e-5) / float(inv_sqrt_d(128)) + 1e-6)


def test_smoothing_shrinks_k_range():
    # the purpose of smoothing ([SA] §3 Figure 4): a shared channel bias is removed
    inp = make_inputs(small(N=512, d=64, seed=8, extras="kbias4"))
    with_s = smooth_quant_qk(inp.qf, inp.kf, smooth=True)["k_scale"]
    without = smooth_quant_qk(inp.qf, inp.kf, smooth=False)["k_scale"]
    assert np.all(with_s < without)


def test_s_int32_exact_vs_int64():
    rng = np.random.default_rng(2)
    qa = rng.integers(-127, 128, size=(1, 1, 96, 128)).astype(np.int8)
    ka = rng.integers(-127, 128, size=(1, 1, 80, 128)).astype(np.int8)
    qa[0, 0, 0] = 127
    ka[0, 0, 0] = 127          # the largest possible magnitude 127*127*128
    s = s_int32_tile(qa, ka, 0, 0, 0, 96, 0, 80)
    ref = np.einsum("nd,md->nm", qa[0, 0].astype(np.int64), ka[0, 0].astype(np.int64))
    assert s.dtype == np.int32
    np.testing.assert_array_equal(s.astype(np.int64), ref)
    assert ref[0, 0] == 127 * 127 * 128


def test_prep_v_fp8_exact_construction():
    # V columns built from E4M3 values times a power of two, each column holding
    # +-448 * 2^e: then r = 2^-e exactly, the codes reproduce the values and
    # decoded * delta_V = V exactly (delta_V = colmax/448 per channel).
    rng = np.random.default_rng(3)
    N, d = 100, 16
    codes = rng.integers(0, 0x7F, size=(1, 1, N, d)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7)
    codes[0, 0, 7, :] = 0x7E
    e = rng.integers(-4, 5, size=d)
    v = (e4m3_decode(codes) * np.ldexp(1.0, e)[None, None, None, :]).astype(np.float32)
    vals, vcodes, vscale = prep_v(v, "fp8")
    np.testing.assert_array_equal(vals * vscale[:, :, None, :].astype(np.float64), v)
    np.testing.assert_array_equal(vscale[0, 0], (448.0 * np.ldexp(1.0, e) / 448.0).astype(np.float32))


def test_prep_v_fp8_error_bound_and_fp16():
    inp = make_inputs(small(N=700, d=64, seed=9))
    vals, codes, vscale = prep_v(inp.vf, "fp8")
    assert codes.dtype == np.uint8
    rec = vals * vscale[:, :, None, :]
    # E4M3 relative half-ulp is 2^-4 for normal values; subnormal step 2^-9 * delta_V
    tol = np.maximum(np.abs(inp.vf) * 2.0 ** -4, 2.0 ** -10 * vscale[:, :, None, :]) * (1 + 1e-6)
    assert np.all(np.abs(rec - inp.vf) <= tol)
    assert np.all(np.abs(vals) <= 448.0)
    assert np.all(np.abs(vals).max(axis=2) == 448.0)        # colmax maps to 448
    v16, _, s = prep_v(inp.vf, "fp16")
    assert s is None
    np.testing.assert_array_equal(v16, inp.vf.astype(np.float16).astype(np.float64))


def test_prep_v_int8_hand_worked():
    # channel 0: colmax 1 -> r = 127, V r = [127, -63.5, 31.75, 95.25] ->
    # codes [127, -64 (tie to even), 32, 95], delta_V = fp32(1/127);
    # channel 1 all zero -> codes 0, delta_V = 0; channel 2: colmax 2.54 ->
    # r = fp32(127/2.54) = 50, codes of [-2.54, 1.27, 0.01, 0] = [-127, 64 (63.5
    # ties to even), 0 (0.5 ties to even), 0]
    v = np.array([[1.0, 0.0, -2.54], [-0.5, 0.0, 1.27], [0.25, 0.0, 0.01],
                  [0.75, 0.0, 0.0]], dtype=np.float32)[None, None]
    vals, codes, vscale = prep_v(v, "int8")
    assert codes.dtype == np.int8
    r2 = np.float32(np.float32(127.0) / np.float32(2.54))
    exp2 = np.clip(np.rint((v[0, 0, :, 2] * r2).astype(np.float32)), -127, 127)
    np.testing.assert_array_equal(codes[0, 0, :, 0], [127, -64, 32, 95])
    np.testing.assert_array_equal(codes[0, 0, :, 1], [0, 0, 0, 0])
    np.testing.assert_array_equal(codes[0, 0, :, 2], exp2)
    assert codes[0, 0, 0, 2] == -127
    np.testing.assert_array_equal(vals, codes.astype(np.float64))
    np.testing.assert_array_equal(vscale[0, 0], np.array([1.0, 0.0, 2.54], np.float32) / np.float32(127))


def test_prep_v_int8_closed_forms():
    inp = make_inputs(small(N=700, d=64, seed=10))
    vals, codes, vscale = prep_v(inp.vf, "int8")
    cm = np.abs(inp.vf).max(axis=2)
    r = (np.float32(127.0) / cm).astype(np.float32)
    x = (inp.vf * r[:, :, None, :]).astype(np.float64)
    assert np.all(np.abs(x - codes) <= 0.5)                          # nearest integer
    assert np.all(np.abs(codes).max(axis=2) == 127)                  # colmax -> 127
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)
    rec = codes * vscale[:, :, None, :].astype(np.float64)
    # half a step, plus the float32 rounding of r and delta_V (r delta_V != 1)
    tol = 0.5 * vscale[:, :, None, :].astype(np.float64) + np.abs(inp.vf) * 2.0 ** -21
    assert np.all(np.abs(rec - inp.vf) <= tol)
