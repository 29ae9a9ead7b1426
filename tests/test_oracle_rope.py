"""Pins of the oracle's rotary embedding (the step the prepass fuses ahead of
quantisation: "SageAttention ..." detail page, §7 key implementation details,
item 1).  The pages do not print RoPE; the oracle takes the rotate-half form
(channel i pairs with i + d/2).  These checks fix that reading and its
arithmetic against properties that do not depend on the formula as typed.
"""
import numpy as np
import pytest

import oracle
from workloads import rope_tables


def test_identity_tables_leave_x_unchanged():
    x = np.random.default_rng(1).standard_normal((1, 2, 7, 64)).astype(np.float32)
    c = np.ones((7, 32), np.float32)
    s = np.zeros((7, 32), np.float32)
    np.testing.assert_array_equal(oracle.rope_rotate_half(x, c, s), x)


def test_hand_worked_pair_and_pairing():
    # one pair (channel 0 with channel d/2 = 4), exactly representable values:
    # y0 = 3*0.5 - 4*0.75 = -1.5, y4 = 4*0.5 + 3*0.75 = 4.25
    x = np.zeros((1, 1, 1, 8), np.float32)
    x[..., 0], x[..., 4] = 3.0, 4.0
    c = np.full((1, 4), 0.5, np.float32)
    s = np.full((1, 4), 0.75, np.float32)
    y = oracle.rope_rotate_half(x, c, s)
    expect = np.zeros(8, np.float32)
    expect[0], expect[4] = -1.5, 4.25
    np.testing.assert_array_equal(y[0, 0, 0], expect)
    # a quarter turn moves channel 1 into channel 1 + d/2 (not into channel 2)
    x = np.zeros((1, 1, 1, 8), np.float32)
    x[..., 1] = 1.0
    y = oracle.rope_rotate_half(x, np.zeros((1, 4), np.float32), np.ones((1, 4), np.float32))
    assert y[0, 0, 0, 5] == 1.0 and np.count_nonzero(y) == 1


def test_pair_norms_preserved():
    N, d = 300, 128
    c, s = rope_tables(N, d)
    x = np.random.default_rng(2).standard_normal((1, 2, N, d)).astype(np.float32)
    y = oracle.rope_rotate_half(x, c, s).astype(np.float64)
    xd = x.astype(np.float64)
    n_in = xd[..., :d // 2] ** 2 + xd[..., d // 2:] ** 2
    n_out = y[..., :d // 2] ** 2 + y[..., d // 2:] ** 2
    # float32 tables (cos^2 + sin^2 = 1 within 2^-23) and float32 rounding
    np.testing.assert_allclose(n_out, n_in, rtol=3e-6, atol=1e-6)


@pytest.mark.parametrize("shift", [1, 37, 500])
def test_scores_depend_on_relative_position_only(shift):
    d = 64
    rng = np.random.default_rng(3)
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal(d).astype(np.float32)
    N = 600
    c, s = rope_tables(N, d)
    Q = np.broadcast_to(q, (1, 1, N, d)).copy()
    K = np.broadcast_to(k, (1, 1, N, d)).copy()
    rq = oracle.rope_rotate_half(Q, c, s)[0, 0].astype(np.float64)
    rk = oracle.rope_rotate_half(K, c, s)[0, 0].astype(np.float64)
    for t1, t2 in [(5, 2), (40, 90), (3, 3)]:
        a = rq[t1] @ rk[t2]
        b = rq[t1 + shift] @ rk[t2 + shift]
        assert abs(a - b) <= 1e-4 * (np.abs(q).sum() * np.abs(k).sum()) ** 0.5


def test_rope_then_quantised_attention_matches_exact_attention():
    # with the identity quantiser the whole pipeline on rotated inputs is
    # exact softmax attention of the rotated Q, K (smoothing included)
    N, d = 150, 64
    c, s = rope_tables(N, d)
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2, N, d)).astype(np.float32) for _ in range(3))
    k += rng.standard_normal((1, 2, 1, d)).astype(np.float32) * 4
    qr, kr = oracle.rope_rotate_half(q, c, s), oracle.rope_rotate_half(k, c, s)
    for causal in (False, True):
        got = oracle.sage_attention(qr, kr, v, causal=causal, pv_mode="none", quant="none")
        ref = oracle.brute_attention(qr, kr, v, causal=causal)
        assert np.abs(got - ref).max() <= 1e-12
