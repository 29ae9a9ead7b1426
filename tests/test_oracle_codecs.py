"""Pins for the oracle's number codecs and for the input generator's rounding.

E4M3FN facts come from the OCP 8-bit floating point format definition
(bias 7, 3 mantissa bits, max finite 448, smallest subnormal 2^-9); 448 is
also the FP8 range in the SageAttention2++ review page, section 三, core
formulas.  torch's CPU float8_e4m3fn cast is an independent library routine
(round to nearest even; it is compared only where both saturate identically,
|x| <= 464).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_decode, e4m3_encode, fp16_round
from workloads import bf16_bits_to_f32, round_to_bf16_bits

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def torch_e4m3_codes(x):
    t = torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_known_points():
    # (value, code) pairs from the format definition
    cases = [(448.0, 0x7E), (-448.0, 0xFE), (1.0, 0x38), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
             (0.0, 0x00), (-0.0, 0x80), (1.125, 0x39), (240.0, 0x77), (256.0, 0x78),
             # ties to even
             (1.0625, 0x38), (1.1875, 0x3A), (0.5 * 2.0 ** -9, 0x00), (1.5 * 2.0 ** -9, 0x02),
             # saturation: 464 is the tie between 448 and the (absent) 480; anything above -> 448
             (464.0, 0x7E), (1.0e4, 0x7E), (-3.0e38, 0xFE)]
    for v, c in cases:
        assert int(e4m3_encode(np.array([v]))[0]) == c, (v, hex(c))
    assert GOLD["fp8_range"]["value"] == e4m3_decode(np.array([0x7E]))[0]


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert len(codes) == 254
    vals = e4m3_decode(codes)
    back = e4m3_encode(vals)
    # +0 and -0 both round-trip to themselves
    np.testing.assert_array_equal(back, codes)
    # decode agrees with torch's float8 -> float32
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    np.testing.assert_array_equal(vals.astype(np.float32), tv)


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(5)
    xs = [rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 0.05, 1, 30, 150)]
    xs.append(rng.uniform(-464, 464, 200000).astype(np.float32))
    # every midpoint between adjacent finite codes (ties) and its neighbours
    pos = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    xs += [mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, np.float32(1e9))]
    x = np.concatenate(xs).astype(np.float32)
    x = x[np.abs(x) <= 464.0]          # above 464 torch returns NaN, ours saturates
    np.testing.assert_array_equal(e4m3_encode(x), torch_e4m3_codes(x))
    big = np.array([464.5, 500.0, 1e6, -470.0], np.float32)
    np.testing.assert_array_equal(e4m3_encode(big), [0x7E, 0x7E, 0x7E, 0xFE])


def test_fp16_round_matches_torch():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (1e-6, 1e-3, 1, 1e3)])
    ours = fp16_round(x.astype(np.float32))
    ref = torch.from_numpy(x.astype(np.float32)).half().double().numpy()
    np.testing.assert_array_equal(ours, ref)


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # exact ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = bf16_bits_to_f32(round_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("v", [1.0, 0.5, 0.25])
def test_static_p_scale_maps_max_to_top_code(v):
    # max P~ = 1 with delta_P = 1/448 lands exactly on the largest finite code
    assert GOLD["p_tilde_max"]["value"] == 1.0
    code = e4m3_encode(np.array([448.0 * v]))[0]
    assert e4m3_decode(np.array([code]))[0] == 448.0 * v


def test_e4m3_flip_step_hand_values():
    """e4m3_flip_step: the decoded-value change of rounding to the other
    neighbouring code, for values within a relative distance of a boundary."""
    from oracle.codecs import e4m3_flip_step
    y = np.array([17.0,      # the 16/18 boundary itself (ties to even -> 16): step 2
                  17.01,     # within 1e-3 of 17, rounds to 18: step 2 (back to 16)
                  17.1,      # 0.1 away from 17 > 1e-3 * 17.1: no step
                  432.0,     # the 416/448 boundary: step 32
                  448.0,     # top code; its lower boundary 432 is far: no step
                  0.0,       # zero: no step
                  2.0 ** -10,  # the 0 / 2^-9 boundary (ties to even -> 0): step 2^-9
                  1.0])      # exactly representable, boundaries at 0.96875 / 1.0625
    got = e4m3_flip_step(y, 1e-3)
    np.testing.assert_array_equal(got, [2.0, 2.0, 0.0, 32.0, 0.0, 0.0, 2.0 ** -9, 0.0])
    # a relative distance array is applied element by element
    got = e4m3_flip_step(np.array([17.05, 17.05]), np.array([1e-3, 5e-3]))
    np.testing.assert_array_equal(got, [0.0, 2.0])


def test_int8_flip_step_hand_values():
    """int8_flip_step: 1 where y (127 P~, rounded to an integer code in
    [0, 127], ties to even) lies within a relative distance of a half-integer
    between two codes, else 0."""
    from oracle.codecs import int8_flip_step
    y = np.array([2.5,       # a midpoint itself (ties to even -> 2): step
                  2.501,     # 0.001 from 2.5 <= 1e-3 * 2.501: step
                  2.6,       # 0.1 from 2.5: no step
                  127.0,     # top code; its lower midpoint 126.5 is far: no step
                  0.0,       # zero: no step
                  0.4999,    # 1e-4 from the 0/1 midpoint: step
                  3.0])      # an integer: no step
    got = int8_flip_step(y, 1e-3)
    np.testing.assert_array_equal(got, [1.0, 1.0, 0.0, 0.0, 0.0, 1.0, 0.0])
    # a relative distance array is applied element by element; near the top
    # code only the lower midpoint counts (no code above 127)
    got = int8_flip_step(np.array([126.99, 126.99, 127.45]), np.array([1e-3, 1e-2, 1e-3]))
    np.testing.assert_array_equal(got, [0.0, 1.0, 0.0])
