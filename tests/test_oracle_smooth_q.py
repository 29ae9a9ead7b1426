"""Pins for the oracle's smoothing of Q (the optional SageAttention2 step).

"SageAttention2" abstract page: smoothing Q improves the accuracy of the
quantised QK^T; "SageAttention2++ ..." review page, section 三: Q and K are
smoothed before quantisation.  The pages give no formula.  The reading the
oracle implements (its module docstring): per 128-token block the mean qbar of
Q' = Q/sqrt(d) is removed before quantisation, kept per channel as an integer
w on a grid 2^8 finer than the codes, and restored through the compensation
C = rne((w . K^) / 2^8) added to the INT32 product.  What pins it:

* block means: exact on integer inputs, ragged last block divides by its own
  token count;
* zero-mean blocks: smoothing changes nothing (codes, scales bit-identical);
* a lossless construction (each block = a bias vector plus integer codes
  times a power of two): smoothed INT8 attention equals textbook attention,
  where the unsmoothed quantiser is lossy;
* C by int64 brute force, with hand-worked ties of the rounding;
* the guard and the constant-block case fall back to the unsmoothed quantiser;
* on a Q with a per-channel bias shared by all tokens, accuracy improves.
"""
import numpy as np
import pytest

import oracle
from oracle import (Q_BLOCK, SQ_FRAC_BITS, SQ_LIMIT, brute_attention, cos_sim, q_block_mean,
                    q_compensation, quantize_int8_blocks, rel_l1, sage_attention,
                    smooth_quant_qk, smooth_quantize_q_blocks)
from workloads import make_inputs, small


def test_block_mean_exact_and_ragged():
    # integer values: every float32 partial sum is exact; block 1 of N = 130
    # holds 2 tokens and divides by 2
    rng = np.random.default_rng(1)
    q = rng.integers(-50, 51, size=(1, 2, 130, 8)).astype(np.float32)
    m = q_block_mean(q)
    assert m.shape == (1, 2, 2, 8)
    np.testing.assert_array_equal(m[:, :, 0], (q[:, :, :128].astype(np.float64).sum(axis=2)
                                               / 128).astype(np.float32))
    np.testing.assert_array_equal(m[:, :, 1], (q[:, :, 128:].astype(np.float64).sum(axis=2)
                                               / 2).astype(np.float32))
    one = np.full((1, 1, 1, 4), 3.0, np.float32)
    np.testing.assert_array_equal(q_block_mean(one), one)


def test_compensation_brute_force_and_ties():
    # C = rne(P / 256) for the exact integer P = w . K^; hand-worked ties:
    # 1.5 -> 2, 2.5 -> 2, -1.5 -> -2, -2.5 -> -2, -0.5 -> 0, 0.5 -> 0,
    # 383/256 -> 1, -129/256 -> -1
    P = np.array([384, 640, -384, -640, -128, 128, 383, -129, 0, 2 ** 29], np.int64)
    w = P.reshape(1, 1, -1, 1).astype(np.int32)          # one channel, K^ = 1
    k = np.ones((1, 1, 1, 1), np.int8)
    c = q_compensation(w, k)[0, 0, :, 0]
    np.testing.assert_array_equal(c, [2, 2, -2, -2, 0, 0, 1, -1, 0, 2 ** 21])
    # random blocks against an int64 loop
    rng = np.random.default_rng(2)
    w = rng.integers(-20000, 20001, size=(1, 2, 3, 16)).astype(np.int32)
    k = rng.integers(-127, 128, size=(1, 2, 37, 16)).astype(np.int8)
    got = q_compensation(w, k)
    for h in range(2):
        for qb in range(3):
            for t in range(37):
                p = sum(int(w[0, h, qb, c]) * int(k[0, h, t, c]) for c in range(16))
                # round half to even, written from the definition
                fl = p // 256
                rem = p - fl * 256
                ref = fl + (1 if rem > 128 or (rem == 128 and fl % 2 == 1) else 0)
                assert got[0, h, qb, t] == ref


def test_zero_mean_blocks_change_nothing():
    # blocks made of a half and its negation (integers times 2^-10, so every
    # float32 partial sum is exact) have mean 0 exactly: the smoothed
    # quantiser is the plain one, w = 0 and C = 0
    rng = np.random.default_rng(3)
    N, d = 256 + 64, 32
    q = np.zeros((1, 1, N, d), np.float32)
    for j in range(0, N, Q_BLOCK):
        n = min(Q_BLOCK, N - j)
        half = (rng.integers(-3000, 3001, size=(n // 2, d)) * 2.0 ** -10).astype(np.float32)
        q[0, 0, j:j + n // 2] = half
        q[0, 0, j + n // 2:j + 2 * (n // 2)] = -half
    codes, delta, qbar, w, ok = smooth_quantize_q_blocks(q)
    pc, pd = quantize_int8_blocks(q, Q_BLOCK)
    assert np.all(ok) and np.all(qbar == 0) and np.all(w == 0)
    np.testing.assert_array_equal(codes, pc)
    np.testing.assert_array_equal(delta.view(np.uint32), pd.view(np.uint32))


def _lossless_smooth_case(N=256, d=64, seed=4):
    """Q' = b_i + c * 2^-e per 128-token block i: integer codes c with zero
    mean in every block (a half and its negation) and one |c| = 127, a bias b_i
    that is an integer (|b| <= 200, inside the guard) times 2^-e.  Then
    qbar = b_i, a = 127 * 2^-e exactly, r = 2^e, the codes are recovered,
    w = b_i 2^(e+8) is a multiple of 2^8 and C = w K^ / 2^8 is exact:
    smoothed INT8 QK^T is lossless.  K: integers times a power of two per
    64-token block, each block a half and its negation (mean 0, lossless)."""
    rng = np.random.default_rng(seed)
    qs = np.zeros((N, d))
    for j in range(0, N, Q_BLOCK):
        e = 4 + (j // Q_BLOCK) % 2
        half = rng.integers(-127, 128, size=(Q_BLOCK // 2, d))
        half[0, 0] = 127
        c = np.concatenate([half, -half])
        b = rng.integers(-200, 201, size=d) * 2.0 ** -e
        qs[j:j + Q_BLOCK] = b + c * 2.0 ** -e
    k = np.zeros((N, d))
    for j in range(0, N, 64):
        half = rng.integers(-127, 128, size=(32, d)).astype(np.float64)
        half[0, 0] = 127
        k[j:j + 64] = np.concatenate([half, -half]) * 2.0 ** (-(j // 64) % 3)
    qf = (qs * 8.0).astype(np.float32)[None, None]          # Q/sqrt(64) = qs exactly
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    return qf, k.astype(np.float32)[None, None], v


@pytest.mark.parametrize("causal", [False, True])
def test_lossless_construction_equals_textbook(causal):
    qf, kf, vf = _lossless_smooth_case()
    pq = smooth_quant_qk(qf, kf, smooth_q=True)
    assert np.all(pq["q_smoothed"]) and np.all(pq["k_mean"] == 0)
    o = sage_attention(qf, kf, vf, causal=causal, pv_mode="none", prep=pq)
    ref = brute_attention(qf, kf, vf, causal=causal)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # the unsmoothed quantiser of the same Q is lossy here (the bias widens
    # each block's range), so the construction tells the two apart
    o_plain = sage_attention(qf, kf, vf, causal=causal, pv_mode="none")
    assert np.abs(o_plain - ref).max() > 1e-6


def test_guard_and_constant_block_fall_back():
    rng = np.random.default_rng(5)
    N, d = 3 * Q_BLOCK, 64
    q = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    q[0, 0, :Q_BLOCK] = q[0, 0, :Q_BLOCK] * np.float32(1e-4) + np.float32(50.0)   # mean >> spread
    q[0, 0, Q_BLOCK:2 * Q_BLOCK] = np.float32(0.75)                          # constant block
    codes, delta, qbar, w, ok = smooth_quantize_q_blocks(q)
    pc, pd = quantize_int8_blocks(q, Q_BLOCK)
    assert ok.tolist() == [[[False, False, True]]]
    # block 0 would need 127 sum|w| far above the limit
    qt = (q[0, 0, :Q_BLOCK] - q_block_mean(q)[0, 0, 0]).astype(np.float32)
    r0 = np.float32(127.0) / np.abs(qt).max()
    assert 127 * np.abs(np.rint(q_block_mean(q)[0, 0, 0] * r0 * 2.0 ** SQ_FRAC_BITS)).sum() > SQ_LIMIT
    for blk in (0, 1):
        sl = slice(blk * Q_BLOCK, (blk + 1) * Q_BLOCK)
        np.testing.assert_array_equal(codes[0, 0, sl], pc[0, 0, sl])
        assert delta[0, 0, blk] == pd[0, 0, blk] and np.all(w[0, 0, blk] == 0)
        assert np.all(qbar[0, 0, blk] == 0)


def test_smoothing_q_improves_accuracy_on_shared_q_bias():
    # Q with a per-channel bias shared by all tokens (as K in [SA] §3 Figure 4)
    inp = make_inputs(small(N=1024, d=64, H=2, seed=3, extras="qbias4_kbias4"))
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=False)
    on = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none", smooth_q=True)
    off = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none")
    assert rel_l1(on, ref) < 0.9 * rel_l1(off, ref)
    assert cos_sim(on, ref) > cos_sim(off, ref)
    # and it costs nothing measurable where Q has no shared bias
    inp = make_inputs(small(N=1024, d=128, H=2, seed=3, extras="q8_kbias5"))
    ref = brute_attention(inp.qf, inp.kf, inp.vf, causal=False)
    on = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none", smooth_q=True)
    off = sage_attention(inp.qf, inp.kf, inp.vf, causal=False, pv_mode="none")
    assert rel_l1(on, ref) <= rel_l1(off, ref) * 1.01


def test_smoothed_scores_within_quantisation_bound():
    # |S_smoothed - S_exact| <= delta_Q~ delta_K (0.5 sum|K^| + 0.5 + sum|w|/2^9 ...)
    # checked in its simplest sufficient form: the Q side of the error is at
    # most one code step per channel (the codes' half step plus w's rounding
    # 2^-9 and C's half unit), the K side at most half a K step per channel.
    inp = make_inputs(small(N=300, d=64, H=1, seed=6, extras="qbias4_kbias4"))
    pq = smooth_quant_qk(inp.qf, inp.kf, smooth_q=True)
    qs = (inp.qf * oracle.inv_sqrt_d(64)).astype(np.float64)[0, 0]
    ks = (inp.kf - pq["k_mean"][:, :, None, :]).astype(np.float32).astype(np.float64)[0, 0]
    exact = qs @ ks.T
    dq = pq["q_scale"][0, 0][np.arange(300) // 128][:, None].astype(np.float64)
    dk = pq["k_scale"][0, 0][np.arange(300) // 64][None, :].astype(np.float64)
    s = (pq["q_i8"][0, 0].astype(np.float64) @ pq["k_i8"][0, 0].astype(np.float64).T
         + pq["q_comp"][0, 0][np.arange(300) // 128]) * dq * dk
    kdeq = pq["k_i8"][0, 0].astype(np.float64) * dk.T
    bound = (dq * (np.abs(kdeq).sum(axis=1)[None, :] + dk)
             + 0.5 * dk * np.abs(qs).sum(axis=1)[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(s - exact) <= bound)
