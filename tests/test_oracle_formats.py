"""Pins of the oracle's number formats and quantiser (CPU only).

What pins what:
  - the E2M1 and E4M3 value tables against their bit-field definitions (the
    Attn-QAT page's count of 15 distinct FP4 values and the hyperion-consulting.io
    article's split of FP4 into 2 exponent bits and 1 mantissa bit; OCP for
    E4M3 and E8M0);
  - E2M1 and E4M3 rounding against brute-force nearest-value search, with
    exact rational arithmetic on a sample;
  - the MX exponent against the property that the scaled group maximum
    lands in [4, 8);
  - fp16 decode/round against numpy's IEEE conversions;
  - the quantiser against exact round trips, scale covariance and the byte
    footprint the ThriftAttention pages give for the dual KV cache (+28%).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table_from_bits(oracle):
    vals = [oracle.e2m1_value(c) for c in range(16)]
    np.testing.assert_array_equal(np.array(vals), pins.e2m1_values_from_bits())
    pages = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    distinct = {abs(v) if v == 0 else v for v in vals}
    assert len(distinct) == pages["fp4_distinct_values"]["value"]


def test_e4m3_table_from_bits(oracle):
    vals = np.array([oracle.e4m3_value(c) for c in range(127)])
    np.testing.assert_array_equal(vals, pins.E4M3_POS)
    assert vals.max() == 448.0
    assert np.isnan(oracle.e4m3_value(0x7F))
    assert oracle.e4m3_value(0x80 | 0x39) == -pins.E4M3_POS[0x39]


def _all_finite_halves():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return h[np.isfinite(h)].astype(np.float64)


@pytest.mark.parametrize("s", [1.0, 2.0 ** -10, 2.0 ** 5, 0.75 * 2.0 ** -3, 3.25 * 0.0123456789,
                               448.0 * 1.1920928955078125e-07])
def test_e2m1_encode_bruteforce(oracle, s):
    # scales: powers of two (MX) and E4M3 x fp32 products (NVFP4-style)
    s = float(np.float64(np.float32(s)))
    x = _all_finite_halves() * (s / 2.0)  # spread the fp16 grid over the code range
    got = oracle.e2m1_encode(x, s)
    want = pins.e2m1_code(x, s)
    np.testing.assert_array_equal(got, want)


def test_e2m1_encode_midpoints_exact(oracle):
    # every midpoint and its neighbours, checked with exact rationals
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rng = np.random.default_rng(7)
    scales = [1.0, 0.5, float(np.float32(rng.random())), float(np.float32(0.1) * 3.5)]
    for s in scales:
        for m in mids:
            for x in (m * s, np.nextafter(m * s, 0), np.nextafter(m * s, 10), -m * s, 7.0 * s, -100 * s):
                got = oracle.e2m1_encode(np.array([x]), s)[0]
                q = abs(Fraction(float(x)) / Fraction(s))
                best = min(range(8), key=lambda c: (abs(q - Fraction(pins.E2M1_POS[c])), c % 2))
                assert got == best | (8 if np.signbit(x) else 0), (x, s, got, best)


def test_e2m1_negative_zero(oracle):
    assert oracle.e2m1_encode(np.array([-0.0, -0.1, 0.0]), 1.0).tolist() == [8, 8, 0]


def test_e4m3_encode_bruteforce(oracle):
    rng = np.random.default_rng(3)
    # ratios over the whole E4M3 range, with midpoints and saturation
    q = np.concatenate([
        np.exp2(rng.uniform(-14, 10, 200000)),
        (pins.E4M3_POS[:-1] + pins.E4M3_POS[1:]) / 2,
        pins.E4M3_POS,
        np.array([0.0, 448.0, 464.0, 480.0, 1e6, 2.0 ** -11, 3 * 2.0 ** -11]),
    ])
    den = 6.0 * np.float32(rng.uniform(0.01, 2.0, q.size)).astype(np.float64)
    num = q * den
    got = oracle.e4m3_encode_ratio(num, den)
    want = pins.nearest_code(num / den, pins.E4M3_POS)
    # num/den is rounded in fp64 here; verify disagreements exactly
    bad = np.nonzero(got != want)[0]
    for t in bad:
        r = Fraction(float(num[t])) / Fraction(float(den[t]))
        best = min(range(127), key=lambda c: (abs(r - Fraction(float(pins.E4M3_POS[c]))), c % 2))
        assert got[t] == best, (num[t], den[t], got[t], best)
    assert len(bad) < 10


def test_mx_exponent_property(oracle):
    rng = np.random.default_rng(5)
    for amax in np.concatenate([np.exp2(rng.uniform(-30, 30, 2000)), 2.0 ** np.arange(-30, 30)]):
        X = oracle.mx_exponent(amax)
        assert 4.0 <= amax / 2.0 ** X < 8.0
    assert oracle.mx_exponent(0.0) == -127
    assert oracle.mx_exponent(2.0 ** -140) == -127
    assert oracle.mx_exponent(2.0 ** 140) == 127


def test_half_decode_all_patterns(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got = oracle.half_to_double(h)
    want = h.astype(np.float64)
    np.testing.assert_array_equal(got, want)


def test_round_to_half_vs_numpy(oracle):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(100000) * np.exp2(rng.uniform(-28, 17, 100000)),
        # exact ties between neighbouring fp16 values
        (np.arange(1, 2000) + 0.5) * 2.0 ** -24,
        (np.arange(1024, 3000) + 0.5) * 2.0 ** -10,
    ])
    x = x[np.abs(x) < 65504]
    np.testing.assert_array_equal(oracle.round_to_half(x), x.astype(np.float16).astype(np.float64))


def _exact_mx_input(rng, S, D):
    """Values code * 2^X with a code of magnitude 4 or 6 in every 32-group, so
    the group maximum fixes X exactly."""
    codes = rng.integers(0, 16, size=(1, 1, S, D))
    codes[..., ::32] = rng.choice([6, 7, 14, 15], size=codes[..., ::32].shape)
    X = rng.integers(-8, 3, size=(1, 1, S, D // 32)).repeat(32, -1)
    x = pins.e2m1_values_from_bits()[codes] * 2.0 ** X
    return x.astype(np.float16), codes, X


def test_mx_quantize_round_trip(oracle):
    rng = np.random.default_rng(1)
    x, codes, X = _exact_mx_input(rng, 96, 64)
    assert np.all(x.astype(np.float64) == pins.e2m1_values_from_bits()[codes] * 2.0 ** X)
    for axis in (oracle.AXIS_D,):
        t = oracle.quantize(x, axis, oracle.MX)
        np.testing.assert_array_equal(oracle.dequantize(t), x.astype(np.float64))
        np.testing.assert_array_equal(t.scales.astype(np.int64), X[..., ::32] + 127)
    # along the sequence: transpose the construction
    xt = np.swapaxes(x, -1, -2).copy()  # S=64, D=96 -> groups of 32 along S
    t = oracle.quantize(xt, oracle.AXIS_S, oracle.MX)
    np.testing.assert_array_equal(oracle.dequantize(t), xt.astype(np.float64))


def test_nvfp4_quantize_round_trip(oracle):
    rng = np.random.default_rng(2)
    S, D, k = 40, 64, 4
    sg = 2.0 ** -k
    blk = rng.choice(pins.E4M3_POS[40:126], size=(S, D // 16))
    blk[0, 0] = 448.0  # the slice maximum 6 * 448 * sg fixes sg exactly
    codes = rng.integers(0, 16, size=(S, D))
    codes[:, ::16] = rng.choice([7, 15], size=codes[:, ::16].shape)  # a 6 in every group
    x = pins.e2m1_values_from_bits()[codes] * np.repeat(blk, 16, -1) * sg
    x16 = x.astype(np.float16)
    assert np.all(x16.astype(np.float64) == x)
    t = oracle.quantize(x16[None, None], oracle.AXIS_D, oracle.NVFP4)
    assert t.tensor_scale[0, 0] == np.float32(sg)
    np.testing.assert_array_equal(oracle.dequantize(t)[0, 0], x)


def test_decode_matches_independent_decoder(oracle):
    rng = np.random.default_rng(9)
    x = (rng.standard_t(3, size=(2, 3, 130, 64)) * 3).astype(np.float16)
    for fmt in (oracle.NVFP4, oracle.MX):
        for axis in (oracle.AXIS_D, oracle.AXIS_S):
            t = oracle.quantize(x, axis, fmt)
            mine = pins.decode_fp4(t.codes, t.scales, t.tensor_scale, fmt, axis, x.shape)
            np.testing.assert_array_equal(oracle.dequantize(t), mine)


def test_quantize_groups_vs_bruteforce(oracle):
    """Every code and block scale re-derived group by group with brute force."""
    rng = np.random.default_rng(4)
    x = (rng.standard_t(3, size=(1, 2, 37, 64)) * np.exp(rng.standard_normal(64))).astype(np.float16)
    xd = x.astype(np.float64)
    for fmt in (oracle.NVFP4, oracle.MX):
        g = 16 if fmt == oracle.NVFP4 else 32
        t = oracle.quantize(x, oracle.AXIS_D, fmt)
        codes = np.stack([t.codes & 0xF, t.codes >> 4], -1).reshape(1, 2, 37, 64)
        for h in range(2):
            sg = float(np.float32(np.abs(xd[0, h]).max() / 2688.0))
            if fmt == oracle.NVFP4:
                assert t.tensor_scale[0, h] == np.float32(sg)
            for s in range(37):
                for gi in range(64 // g):
                    seg = xd[0, h, s, gi * g:(gi + 1) * g]
                    if fmt == oracle.NVFP4:
                        sb = pins.nearest_code(np.abs(seg).max() / (6 * sg), pins.E4M3_POS)
                        scale = pins.E4M3_POS[sb] * sg
                    else:
                        X = int(pins.mx_exponent(np.abs(seg).max()))
                        sb, scale = X + 127, 2.0 ** X
                    assert t.scales[0, h, s, gi] == sb
                    want = pins.e2m1_code(seg, scale) if scale > 0 else np.zeros(g, int)
                    np.testing.assert_array_equal(codes[0, h, s, gi * g:(gi + 1) * g], want)


@pytest.mark.parametrize("n", [-3, 2, 5])
def test_scale_covariance(oracle, n):
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((1, 2, 64, 64)) * 4).astype(np.float16)
    y = (x.astype(np.float64) * 2.0 ** n).astype(np.float16)
    assert np.all(y.astype(np.float64) == x.astype(np.float64) * 2.0 ** n)
    a, b = oracle.quantize(x, 0, oracle.MX), oracle.quantize(y, 0, oracle.MX)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales.astype(int) + n, b.scales.astype(int))
    a, b = oracle.quantize(x, 0, oracle.NVFP4), oracle.quantize(y, 0, oracle.NVFP4)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales, b.scales)
    np.testing.assert_array_equal(a.tensor_scale * np.float32(2.0 ** n), b.tensor_scale)


def test_dual_cache_footprint(oracle):
    """The pages give +28% KV memory for keeping FP16 and NVFP4 copies."""
    pages = json.load(open(os.path.join(GOLDEN, "pages_numbers.json")))
    rng = np.random.default_rng(0)
    S, D = 256, 128
    x = rng.standard_normal((1, 2, S, D)).astype(np.float16)
    for fmt, ratio in ((oracle.NVFP4, 0.28125), (oracle.MX, 0.265625)):
        k = oracle.quantize(x, oracle.AXIS_D, fmt)
        v = oracle.quantize(x, oracle.AXIS_S, fmt)
        fp4_bytes = k.codes.nbytes + k.scales.nbytes + v.codes.nbytes + v.scales.nbytes
        assert fp4_bytes / (2 * x.nbytes) == ratio
    assert round(100 * 0.28125) == pages["dual_cache_overhead_percent"]["value"]
    # NVFP4 vs FP8: 1 byte against 0.5 + 1/16 bytes per element
    assert round(1.0 / 0.5625, 1) == pages["nvfp4_vs_fp8_size_ratio"]["value"]
    # 131072 tokens x 128 channels of fp16 K and V per head
    assert round(131072 * 128 * 2 * 2 / 2 ** 20) == pages["kv_fp16_mb_per_head_131k"]["value"]
