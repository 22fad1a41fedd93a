"""Pins of the oracle's bf16 rounding (round_f64_to_bf16) against hand-derived values.

tests/golden/bf16_round_cases.json lists inputs and the nearest bf16 value worked out by
hand from the format (7 stored mantissa bits, exponent range of fp32, subnormals m *
2^-133) with ties to even: ties in both directions, values just off a tie (including
offsets finer than fp32, which a rounding through fp32 would lose), the exponent and
subnormal/normal boundaries, the smallest subnormal, overflow to infinity and signed
zero.  Truncation, ties away from zero or a double rounding through fp32 each fail
several of them.
"""
import json
import os

import numpy as np

from oracle.numerics import bf16_value_to_bits, round_f64_to_bf16

GOLD = os.path.join(os.path.dirname(__file__), "golden", "bf16_round_cases.json")


def _cases():
    d = json.load(open(GOLD))
    xs = np.array([float.fromhex(c["x"]) for c in d["cases"]])
    ys = np.array([np.inf if c["bf16"] == "inf" else float.fromhex(c["bf16"]) for c in d["cases"]])
    return xs, ys, [c["why"] for c in d["cases"]]


def test_round_f64_to_bf16_hand_derived_cases():
    xs, ys, why = _cases()
    got = round_f64_to_bf16(xs)
    for x, y, g, w in zip(xs, ys, got, why):
        assert g == y and np.signbit(g) == np.signbit(y), f"{x!r}: {w}: got {g!r}, want {y!r}"


def test_round_f64_to_bf16_results_are_bf16_values():
    """Every finite result survives the bit-pattern round trip (it is a bf16 value)."""
    xs, _, _ = _cases()
    rng = np.random.default_rng(0)
    xs = np.concatenate([xs, rng.standard_normal(1000) * 10.0 ** rng.integers(-40, 38, 1000)])
    got = round_f64_to_bf16(xs)
    fin = np.isfinite(got)
    back = (bf16_value_to_bits(got[fin]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(back, got[fin])
