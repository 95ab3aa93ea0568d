"""Pins of the oracle's E4M3 / BF16 codecs against facts the pages and the format fix.

* TeleFuser "面向注意力的 FP8 Preparation": scales divide amax by 448, the largest E4M3 value.
* P-cast paper section 三: 3-bit mantissa, 8 values per binade (12.5 % relative step);
  a P value underflows iff p * S < 2^-10.
* VC-Attention section 三: ExpCast adds 56 (= 8 x bias 7), the code of 1.0.
The encoder is also checked against an independent nearest-value search over the 127
finite non-negative grid points (brute force), and the BF16 encoder against torch.
"""
import math

import numpy as np
import pytest
import torch


def _grid(orc):
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    return codes, orc.e4m3_decode(codes)


def _nearest_even(vals, x):
    """Brute-force RNE onto the grid: nearest value, ties to the even code; saturating."""
    a = np.abs(x)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among tied candidates prefer the even code
    codes = np.arange(vals.size)
    even_pref = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 10_000).min(axis=1)
    any_pref = np.where(cand, codes[None, :], 10_000).min(axis=1)
    c = np.where(even_pref < 10_000, even_pref, any_pref).astype(np.uint8)
    c = np.where(a >= 448.0, 0x7E, c).astype(np.uint8)
    return np.where(np.signbit(x), c | 0x80, c).astype(np.uint8)


def test_roundtrip_all_256_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.e4m3_decode(codes)
    nan = np.isnan(vals)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    back = orc.e4m3_encode(vals)
    assert np.array_equal(back[~nan], codes[~nan])      # includes -0 -> 0x80
    assert np.all(back[nan] == 0x7F)
    assert vals[0x38] == 1.0 and vals[0x78] == 256.0 and vals[0x7E] == 448.0
    assert np.nanmax(vals) == 448.0                       # the "/448" of the block scales
    assert vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6


def test_eight_values_per_binade(orc):
    _, vals = _grid(orc)
    for e in range(-6, 8):
        inside = vals[(vals >= 2.0 ** e) & (vals < 2.0 ** (e + 1))]
        assert inside.size == 8
        assert np.allclose(np.diff(inside) / 2.0 ** e, 0.125)   # 12.5 % relative step
    top = vals[vals >= 256.0]
    assert top.size == 7                                     # 448 = 1.75 * 2^8 is the top


def test_underflow_threshold_is_2_pow_minus_10(orc):
    rng = np.random.default_rng(0)
    x = 2.0 ** rng.uniform(-16, -8, 200_000)
    c = orc.e4m3_encode(x)
    assert np.all(c[x < 2.0 ** -10] == 0)
    assert np.all(c[x > 2.0 ** -10] != 0)
    assert orc.e4m3_encode([2.0 ** -10])[0] == 0              # tie -> even code 0
    assert orc.e4m3_encode([np.nextafter(2.0 ** -10, 1.0)])[0] == 0x01


def test_saturation_pins(orc):
    x = [448.0 * (1 + 2.0 ** -23), 448.0, 463.99, 464.0, 465.0, 1e9, math.inf, -1e9]
    assert list(orc.e4m3_encode(x)) == [0x7E] * 7 + [0xFE]
    assert orc.e4m3_encode([math.nan])[0] == 0x7F


def test_encoder_matches_bruteforce_nearest(orc):
    codes, vals = _grid(orc)
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                          np.nextafter(vals, 0), np.nextafter(vals, 1e9)])
    rng = np.random.default_rng(1)
    pts = np.concatenate([pts, 2.0 ** rng.uniform(-14, 9.2, 100_000), [0.0, 500.0, 1e30]])
    pts = np.concatenate([pts, -pts])
    got = orc.e4m3_encode(pts)
    want = _nearest_even(vals, pts)
    assert np.array_equal(got, want)
    # the FP32 entry point agrees with the FP64 one on FP32 inputs
    p32 = pts.astype(np.float32)
    assert np.array_equal(orc.e4m3_encode_f32(p32), orc.e4m3_encode(p32.astype(np.float64)))


def test_expcast_offset_is_code_of_one(orc):
    # ExpCast: c = round(8 z + 56 + beta); 56 = 8 * (exponent bias 7) is the code of 1.0.
    assert orc.e4m3_decode(np.array([56], np.uint8))[0] == 1.0
    # the code of 2^z for integer z in the normal range is 8 z + 56
    z = np.arange(-6, 9)
    assert np.array_equal(orc.e4m3_encode(2.0 ** z), (8 * z + 56).astype(np.uint8))


def test_bf16_encoder_matches_torch(orc):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.uniform(-30, 30, 100_000),
                        [0.0, -0.0, 1.0, 3.0e38]]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_encode(x), want)
    assert np.array_equal(orc.bf16_decode(want), torch.from_numpy(want.view(np.int16)).view(
        torch.bfloat16).float().double().numpy())


@pytest.mark.parametrize("k", range(0, 9))
def test_power_of_two_scaling_is_exact(k):
    # P-cast paper, optimality condition 1: x * 2^k and x * 2^-k are exact in FP32.
    rng = np.random.default_rng(k)
    x = rng.uniform(1e-30, 1.0, 10_000).astype(np.float32)
    S = np.float32(2.0 ** k)
    assert np.array_equal((x * S) / S, x)


def test_scaling_by_448_is_not_exact():
    rng = np.random.default_rng(9)
    x = rng.uniform(1e-6, 1.0, 10_000).astype(np.float32)
    S = np.float32(448.0)
    assert not np.array_equal((x * S) / S, x)
