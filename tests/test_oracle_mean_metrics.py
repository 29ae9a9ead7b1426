"""Pins for two oracle parts that agreement with the GPU cannot check on its
own: the fixed float32 summation order of the K column mean, and the
accuracy metrics.

"SageAttention: Accurate 8-Bit Attention ..." (paper detail page), §4 Eq. 6:
smoothing subtracts the token mean of every K channel.  Any vector subtracted
from every key leaves softmax unchanged, so the page fixes no precision or
order; this library takes one fixed float32 order (256-token chunk partials,
each summed sequentially from 0.0f in token order, then the partials summed
sequentially in chunk order, then one IEEE division by N).  The columns below
are built so that float32 rounding makes that order visible in the result:
a flat sequential sum, another chunk size, a reversed chunk or reversed
partials, or a multiplication by 1/N each give different bits.

§5 Table 2 reports CosSim, Relative L1 and RMSE without defining them; the
oracle takes the usual definitions, checked here on hand-worked vectors.
"""
import math

import numpy as np

from oracle import column_mean, cos_sim, rel_l1, rmse, smooth_quant_qk

TWO24 = np.float32(2.0 ** 24)   # float32 spacing is 2 from here up


def _chunk_order_columns(N=600):
    """float32 [1, 1, N, 2] keys; columns A and B (see the expected values)."""
    k = np.zeros((1, 1, N, 2), np.float32)
    # A: 2^24 then ones.  Inside chunk 0 every +1 meets 2^24 and rounds back
    # to it (tie to even); chunk 1 sums its 256 ones exactly, chunk 2 its 88.
    k[0, 0, 0, 0] = TWO24
    k[0, 0, 1:, 0] = 1.0
    # B: one value per chunk: +2^24, +1, -2^24.  In chunk order the +1 is
    # absorbed by 2^24 and the total is 0; in reverse order it survives.
    k[0, 0, 0, 1] = TWO24
    k[0, 0, 256, 1] = 1.0
    k[0, 0, 512, 1] = -TWO24
    return k


def test_mean_chunk_order_hand_worked():
    k = _chunk_order_columns()
    m = column_mean(k)[0, 0]
    # A: partials 2^24, 256, 88 -> (2^24 + 256) + 88 = 16777560 (exact, even);
    # 16777560 / 600 = 27962.6, float32 spacing 2^-9 there:
    # 27962.6 / 2^-9 = 14316851.2 -> 14316851 * 2^-9 = 27962.599609375
    assert m[0] == np.float32(27962.599609375)
    # B: (2^24 + 1) -> 2^24, then + (-2^24) -> 0
    assert m[1] == np.float32(0.0)
    assert m.dtype == np.float32


def test_mean_chunk_order_discriminates():
    # The expected values above differ from what the plausible wrong orders
    # give, so the pin would catch each of them.
    k = _chunk_order_columns()
    col_a, col_b = k[0, 0, :, 0], k[0, 0, :, 1]
    N = np.float32(col_a.size)

    def seq(xs):
        s = np.float32(0.0)
        for x in xs:
            s = np.float32(s + x)
        return s

    def chunked(xs, size, reverse_parts=False, reverse_inside=False):
        parts = []
        for j in range(0, xs.size, size):
            c = xs[j:j + size]
            parts.append(seq(c[::-1] if reverse_inside else c))
        return seq(parts[::-1] if reverse_parts else parts)

    ok_a = np.float32(27962.599609375)
    assert seq(col_a) / N != ok_a                                     # flat sum
    assert chunked(col_a, 128) / N != ok_a                            # chunk 128
    assert chunked(col_a, 512) / N != ok_a                            # chunk 512
    assert chunked(col_a, 256, reverse_inside=True) / N != ok_a       # reversed chunk
    assert chunked(col_b, 256, reverse_parts=True) / N != np.float32(0.0)   # reversed partials
    assert chunked(col_a, 256) * np.float32(1.0 / 600.0) != ok_a      # times 1/N
    # and the right order reproduces both
    assert chunked(col_a, 256) / N == ok_a
    assert chunked(col_b, 256) / N == np.float32(0.0)


def test_mean_ragged_last_chunk():
    # N = 257: chunk 1 holds one token; its partial is that token exactly.
    k = np.zeros((1, 1, 257, 1), np.float32)
    k[0, 0, 0, 0] = TWO24
    k[0, 0, 1:256, 0] = 1.0      # lost inside chunk 0
    k[0, 0, 256, 0] = 2.0        # chunk 1 = 2 -> total 2^24 + 2
    # (2^24 + 2) / 257 = 65281 + 1/257 = 65281.00389...; float32 spacing 2^-8
    # at [2^15, 2^16): 65281.00389 * 256 = 16711936.996 -> 16711937 / 256
    assert column_mean(k)[0, 0, 0] == np.float32(65281.00390625)
    # one flat sum would lose the 2 as well: 2^24 / 257
    assert TWO24 / np.float32(257) != np.float32(65281.00390625)


def test_smoothed_column_sums_vanish():
    # sum_t (K[t, c] - mean_c) = N (exact_mean - mean_c) plus the float32
    # rounding of each difference: bounded by the mean's own float32 error.
    rng = np.random.default_rng(11)
    N, d = 1000, 64
    k = (rng.standard_normal((1, 2, N, d)) + 5.0 * rng.standard_normal((1, 2, 1, d)))
    k = k.astype(np.float16).astype(np.float32)
    q = rng.standard_normal((1, 2, N, d)).astype(np.float16).astype(np.float32)
    mean = column_mean(k)
    ks = (k - mean[:, :, None, :]).astype(np.float32)
    u = 2.0 ** -24
    for h in range(2):
        for c in range(d):
            col = k[0, h, :, c].astype(np.float64)
            exact = math.fsum(col) / N
            err_mean = abs(exact - float(mean[0, h, c]))
            # a fp32 sum of N terms errs by at most ~N u sum|x| (crude, safe)
            assert err_mean <= 2 * N * u * np.abs(col).sum() / N + u * abs(exact)
            s = math.fsum(ks[0, h, :, c].astype(np.float64))
            bound = N * err_mean + u * np.abs(ks[0, h, :, c]).astype(np.float64).sum() + 1e-12
            assert abs(s) <= bound
    # the smoothed keys the prepass quantises are these differences
    pq = smooth_quant_qk(q, k)
    assert np.array_equal(pq["k_mean"], mean)


def test_rmse_hand_worked():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    ref = np.array([1.0, 0.0, 3.0, 0.0])
    # differences 0, 2, 0, 4; squares 0, 4, 0, 16; mean 5; sqrt 5
    assert rmse(x, ref) == math.sqrt(5.0)
    # flattened over any shape, symmetric
    assert rmse(x.reshape(2, 2), ref.reshape(2, 2)) == math.sqrt(5.0)
    assert rmse(ref, x) == math.sqrt(5.0)
    # one element off by 3 in nine: sqrt(9/9) = 1
    assert rmse(np.full(9, 3.0) * (np.arange(9) == 4), np.zeros(9)) == 1.0


def test_rel_l1_hand_worked():
    x = np.array([1.0, -2.0, 3.0])
    ref = np.array([2.0, -2.0, 1.0])
    # |x - ref| = 1, 0, 2 -> 3; |ref| = 2, 2, 1 -> 5
    assert rel_l1(x, ref) == 3.0 / 5.0
    # normalised by the reference, not by x
    assert rel_l1(ref, x) == 3.0 / 6.0


def test_cos_sim_hand_worked():
    assert cos_sim([3.0, 4.0], [4.0, 3.0]) == 24.0 / 25.0
    assert cos_sim([1.0, 0.0], [0.0, 5.0]) == 0.0
    assert math.isclose(cos_sim([1.0, 2.0], [-2.0, -4.0]), -1.0, rel_tol=0, abs_tol=1e-15)
