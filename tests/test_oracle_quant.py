"""Pins of the oracle's smoothing and quantizers (CPU only).

What pins what:
* hand-derived golden cases (tests/golden/*.json) for the INT4 and FP4 quantizers;
* the defining properties of round-to-nearest and of s = max|v| / q_max, checked in
  exact rational arithmetic (fractions), never by re-running the oracle's formula;
* exhaustive sweeps over every finite bf16 value for both quantizers;
* closed-form special cases of the smoothing factor and the outlier-balancing
  property it is designed for (ch3chohch3.github.io post, "Smooth Quant（W8A8）").
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant
from oracle.numerics import bf16_to_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fr(x):
    return Fraction(float(x))


def _all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        v = bf16_to_f64(b)
    return v[np.isfinite(v)]


# ------------------------------------------------------------------ INT4

def test_int4_golden_cases():
    d = json.load(open(os.path.join(GOLD, "int4_cases.json")))
    for c in d["cases"]:
        vals = np.zeros(64, dtype=np.float32)
        vals[: len(c["values"])] = np.array(c["values"], dtype=np.float32)
        codes, sb = quant.quantize_int4(vals[None, :])
        assert int(sb[0, 0]) == c["scale_bits"], c["why"]
        assert codes[0, : len(c["codes"])].tolist() == c["codes"], c["why"]
        assert not codes[0, len(c["codes"]):].any()
    nb = d["nibble_packing"]
    nib = quant.int4_to_nibble(np.array(nb["codes"], dtype=np.int8))
    assert quant.pack_nibbles(nib).tolist() == nb["bytes"]
    back = quant.nibble_to_int4(quant.unpack_nibbles(np.array(nb["bytes"], dtype=np.uint8)))
    assert back.tolist() == nb["codes"]
    # every code round-trips, and zero is never the negative-zero nibble
    q = np.arange(-7, 8, dtype=np.int8)
    assert np.array_equal(quant.nibble_to_int4(quant.int4_to_nibble(q)), q)
    assert quant.int4_to_nibble(np.int8(0)) == 0


def _check_int4_group_properties(vals32, codes, sbits):
    """Exact checks that q = round(v/s), s = max|v|/7 rounded to fp16, per group."""
    a = max(abs(_fr(v)) for v in vals32)
    s = _fr(np.uint16(sbits).view(np.float16))
    if a == 0:
        assert s == 0 and not np.any(codes)
        return
    # s is within fp16 rounding (plus the fp32 step) of a / 7
    rel = abs(s - a / 7) / (a / 7)
    if s >= Fraction(2) ** -14:  # normal fp16
        assert rel <= Fraction(1, 2 ** 11) * (1 + Fraction(1, 2 ** 20)), (float(a), float(s))
    for v, q in zip(vals32, codes):
        v = _fr(v)
        q = int(q)
        assert -7 <= q <= 7
        t = v / s
        if abs(t) <= 7:
            # nearest integer, ties to even
            d = abs(t - q)
            assert d <= Fraction(1, 2), (float(v), float(s), q)
            if d == Fraction(1, 2):
                assert q % 2 == 0
        else:
            assert q == (7 if t > 0 else -7)


def test_int4_round_to_nearest_property_random_and_ties():
    rng = np.random.default_rng(7)
    for trial in range(300):
        g = rng.standard_normal(64).astype(np.float32) * np.float32(10.0 ** rng.uniform(-6, 4))
        if trial % 3 == 0:
            # plant exact ties v = (n + 1/2) s and near-ties one ulp either side
            _, sb = quant.quantize_int4(g[None, :])
            s = np.float32(np.uint16(sb[0, 0]).view(np.float16))
            for j in range(1, 20):
                n = int(rng.integers(-7, 7))
                v = np.float32((n + 0.5) * float(s))
                if abs(v) < np.abs(g).max():
                    g[j] = [v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))][j % 3]
        codes, sb = quant.quantize_int4(g[None, :])
        _check_int4_group_properties(g, codes[0], sb[0, 0])


def test_int4_absmax_maps_to_qmax_and_symmetry():
    rng = np.random.default_rng(11)
    g = rng.standard_normal((500, 64)).astype(np.float32) * np.float32(3.0)
    codes, sb = quant.quantize_int4(g)
    s = sb.view(np.float16).astype(np.float64)
    assert np.all(s > 2 ** -14)  # normal scales here
    am = np.abs(g).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(500), am]) == 7)
    codes_neg, sb_neg = quant.quantize_int4(-g)
    assert np.array_equal(sb, sb_neg) and np.array_equal(codes_neg, -codes)


def test_int4_exhaustive_bf16_sweep():
    """Every finite bf16 magnitude against several group scales (exact rationals)."""
    v = _all_finite_bf16().astype(np.float32)
    for amax in [1.0, 0.3, 7.0, 1e-3, 123.456, 3e4]:
        amax = np.float32(amax)
        sel = v[np.abs(v) <= amax]
        pad = (-len(sel)) % 63
        sel = np.concatenate([sel, np.zeros(pad, np.float32)]).reshape(-1, 63)
        g = np.concatenate([np.full((sel.shape[0], 1), amax, np.float32), sel], axis=1)
        codes, sb = quant.quantize_int4(g)
        assert len(set(sb[:, 0].tolist())) == 1
        s = _fr(np.uint16(sb[0, 0]).view(np.float16))
        # vectorised exact check: |v - q s| <= s/2 with ties to even, via integer arithmetic
        # v and s are dyadic rationals: scale both to integers with a common power of two
        den = 2 ** 200
        vi = [int(Fraction(float(x)) * den) for x in g.ravel()]
        si = int(s * den)
        qs = codes.ravel().astype(np.int64).tolist()
        for x, q in zip(vi, qs):
            r = x - q * si
            assert 2 * abs(r) <= si or abs(q) == 7
            if 2 * abs(r) == si:
                assert q % 2 == 0


def test_int4_zero_and_tiny_groups():
    codes, sb = quant.quantize_int4(np.zeros((2, 64), np.float32))
    assert not codes.any() and not sb.any()
    tiny = np.full((1, 64), np.float32(1e-8))  # a / 7 underflows fp16 to zero
    codes, sb = quant.quantize_int4(tiny)
    assert sb[0, 0] == 0 and not codes.any()
    sub = np.zeros((1, 64), np.float32)
    sub[0, 0] = np.float32(7 * 2.0 ** -20)  # fp16 subnormal scale, still exact 2^-20
    sub[0, 1] = np.float32(-3.5 * 2.0 ** -20)
    codes, sb = quant.quantize_int4(sub)
    assert np.float16(np.uint16(sb[0, 0]).view(np.float16)) == np.float16(2.0 ** -20)
    assert codes[0, :2].tolist() == [7, -4]


def test_int4_scale_saturates():
    g = np.zeros((1, 64), np.float32)
    g[0, 0] = np.float32(1e6)
    codes, sb = quant.quantize_int4(g)
    assert np.uint16(sb[0, 0]).view(np.float16) == np.float16(65504)
    assert codes[0, 0] == 7  # 1e6 / 65504 = 15.3 clamps to 7


# ------------------------------------------------------------------ FP4

def test_fp4_golden_cases():
    d = json.load(open(os.path.join(GOLD, "fp4_cases.json")))
    t = d["ties"]
    assert quant.e2m1_round(np.array(t["scaled_values"])).tolist() == t["index"]
    e = d["exponent"]
    assert quant.fp4_exponent(np.array(e["absmax"], dtype=np.float32)).tolist() == e["e"]
    g = d["group"]
    vals = np.zeros(32, np.float32)
    vals[: len(g["values"])] = np.array(g["values"], np.float32)
    codes, e8 = quant.quantize_mxfp4(vals[None, :])
    assert int(e8[0, 0]) == g["e8m0"]
    assert codes[0, : len(g["codes"])].tolist() == g["codes"]


def test_fp4_exhaustive_bf16_nearest_point():
    """Every finite bf16 value as a group member: grid membership, nearest point,
    ties to even index, |v / 2^e| <= 6, and e minimal (exact rationals)."""
    v = _all_finite_bf16().astype(np.float32)
    grid = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
    for amax in [6.0, 1.0, 0.7, 5.5e-3, 3.0e5]:
        amax = np.float32(amax)
        sel = v[np.abs(v) <= amax]
        # subsample deterministically to keep the exact loop fast, keep the extremes
        sel = sel[:: max(1, len(sel) // 6000)]
        pad = (-len(sel)) % 31
        sel = np.concatenate([sel, np.zeros(pad, np.float32)]).reshape(-1, 31)
        g = np.concatenate([np.full((sel.shape[0], 1), amax, np.float32), sel], axis=1)
        codes, e8 = quant.quantize_mxfp4(g)
        e = int(e8[0, 0]) - 127
        a = _fr(amax)
        assert 6 * Fraction(2) ** e >= a and 6 * Fraction(2) ** (e - 1) < a
        for x, c in zip(g.ravel(), codes.ravel()):
            u = _fr(x) / Fraction(2) ** e
            assert abs(u) <= 6
            idx = int(c) & 7
            assert (int(c) >> 3) == (1 if math.copysign(1.0, float(x)) < 0 else 0)
            d = [abs(abs(u) - gv) for gv in grid]
            best = min(d)
            assert d[idx] == best, (float(x), e, idx)
            if sum(1 for dd in d if dd == best) > 1:
                assert idx % 2 == 0


def test_fp4_absmax_in_3_4_6():
    rng = np.random.default_rng(3)
    g = (rng.standard_normal((400, 32)) * 10.0 ** rng.uniform(-5, 5, (400, 1))).astype(np.float32)
    codes, e8 = quant.quantize_mxfp4(g)
    am = np.abs(g).argmax(axis=1)
    mag = quant.E2M1_GRID[codes[np.arange(400), am] & 7]
    assert set(mag.tolist()) <= {3.0, 4.0, 6.0}


def test_fp4_zero_group():
    codes, e8 = quant.quantize_mxfp4(np.zeros((1, 32), np.float32))
    assert e8[0, 0] == 127 and not codes.any()


# ------------------------------------------------------------------ smoothing

def test_smoothing_closed_forms():
    rng = np.random.default_rng(5)
    a = np.abs(rng.standard_normal(200)) * 30 + 0.01
    w = np.abs(rng.standard_normal(200)) * 3 + 0.01
    s64, s32, inv = quant.smoothing_factors(a, w, 0.5)
    np.testing.assert_allclose(s64, np.sqrt(a / w), rtol=4e-16)
    s64, _, _ = quant.smoothing_factors(a, w, 1.0)
    assert np.array_equal(s64, a)
    s64, _, _ = quant.smoothing_factors(a, w, 0.0)
    np.testing.assert_allclose(s64, 1.0 / w, rtol=2e-16)
    s64, _, _ = quant.smoothing_factors(a, a, 0.75)
    np.testing.assert_allclose(s64, a ** 0.5, rtol=4e-16)  # a = w => s = a^(2 alpha - 1)
    # stored forms: fp32 of s, and the IEEE single reciprocal of that fp32
    _, s32, inv = quant.smoothing_factors(a, w, 0.5)
    for x, y in zip(s32[:50], inv[:50]):
        exact = 1 / _fr(x)
        # nearest fp32 to 1/x: y within half an ulp
        ulp = Fraction(2) ** (math.frexp(float(y))[1] - 24)
        assert abs(_fr(y) - exact) <= ulp / 2


def test_smoothing_zero_channels_floored():
    s64, s32, inv = quant.smoothing_factors(np.array([0.0, 2.0]), np.array([3.0, 0.0]), 0.5)
    assert np.all(np.isfinite(s64)) and np.all(s64 > 0)
    np.testing.assert_allclose(s64, [math.sqrt(1e-5 / 3.0), math.sqrt(2.0 / 1e-5)])


def test_smoothing_identity_and_balance():
    """(X diag(s)^-1)(diag(s) W) = X W, and at alpha = 0.5 each channel's activation
    and weight maxima become equal (sqrt(a w)): the outlier migration smoothing is for."""
    from bit_diffusion_model_amd.workloads import make
    wl = make("C0")
    X = bf16_to_f64(wl.X)
    W = bf16_to_f64(wl.W)
    a = quant.channel_absmax_cols(wl.X)
    w = quant.channel_absmax_rows(wl.W)
    s64, s32, inv = quant.smoothing_factors(a, w, 0.5)
    lhs = (X / s64[None, :]) @ (s64[:, None] * W)
    ref = X @ W
    assert np.abs(lhs - ref).max() <= 1e-12 * np.abs(ref).max()
    xh = np.abs(X / s64[None, :]).max(axis=0)
    wh = np.abs(s64[:, None] * W).max(axis=1)
    np.testing.assert_allclose(xh, wh, rtol=1e-12)
    np.testing.assert_allclose(xh, np.sqrt(a * w), rtol=1e-12)
    # activations become more uniform across channels: the peak-to-median ratio drops
    assert xh.max() / np.median(xh) < 0.5 * (a.max() / np.median(a))


def test_smooth_activations_is_single_fp32_product():
    rng = np.random.default_rng(9)
    from bit_diffusion_model_amd.workloads import bf16_bits_from_f64
    Xb = bf16_bits_from_f64(rng.standard_normal((4, 64)) * 5)
    inv = (rng.uniform(0.1, 3, 64)).astype(np.float32)
    xh = quant.smooth_activations(Xb, inv)
    for i in range(4):
        for j in range(0, 64, 7):
            exact = _fr(bf16_to_f64(Xb[i, j])) * _fr(inv[j])
            y = _fr(xh[i, j])
            if exact != 0:
                ulp = Fraction(2) ** (math.frexp(float(exact))[1] - 24)
                assert abs(y - exact) <= ulp / 2
