"""Pins of the oracle's 4-bit weight-only baseline (oracle/weight_only.py).

* The upcast bf16(s_W q): hand-derived cases (tests/golden/w4a16_upcast_cases.json:
  ties in both directions, values off a tie, the smallest subnormal and the saturated
  fp16 scale), and every positive finite fp16 scale with every code against an integer
  evaluation (the product as an integer times a power of two, rounded to 8 significant
  bits with integer shifts, ties to even): truncation, ties away, a rounding through
  fp16 or a dropped scale each fail.
* The weight quantizer on W: planted columns whose groups are exact multiples of
  distinct fp16 scales give back those codes and scales, in [N][K] / [K/64][N] order, so
  a transposed layout or a group taken along the wrong axis fails.
* The product: a triple loop over a non-square tiny layer (a transposed operand or a
  wrong axis fails), and the reduction to a plain matrix product when every weight is
  already a bf16 value of the form s q.
"""
import json
import os

import numpy as np
import pytest

from oracle import weight_only as wo
from oracle.numerics import bf16_to_f64, bf16_value_to_bits

GOLD = os.path.join(os.path.dirname(__file__), "golden", "w4a16_upcast_cases.json")


def test_upcast_hand_derived_cases():
    d = json.load(open(GOLD))
    for c in d["cases"]:
        sb = np.array([[int(c["s_bits"], 16)]], dtype=np.uint16)
        codes = np.full((1, 64), c["q"], dtype=np.int8)
        got = wo.upcast(codes, sb)
        assert got.shape == (64, 1)
        assert int(got[0, 0]) == int(c["bf16"], 16), f"{c['why']}: got {hex(int(got[0, 0]))}"


def _f16_parts(bits):
    """fp16 bits -> (integer significand m, exponent e) with value m * 2^e (exact)."""
    b = bits.astype(np.int64)
    E = (b >> 10) & 0x1F
    f = b & 0x3FF
    m = np.where(E == 0, f, f | 0x400)
    e = np.where(E == 0, -24, E - 25)
    return m, e


def _round_int_to_bf16_value(Nv, e):
    """Integer Nv > 0 times 2^e rounded to 8 significant bits, ties to even (integers)."""
    L = np.frexp(Nv.astype(np.float64))[1]  # bit length of Nv
    sh = np.maximum(L - 8, 0)
    r = Nv >> sh
    rem = Nv - (r << sh)
    half = np.where(sh > 0, np.left_shift(1, np.maximum(sh - 1, 0)), 0)
    up = (sh > 0) & ((rem > half) | ((rem == half) & (r % 2 == 1)))
    r = r + up
    return np.ldexp(r.astype(np.float64), (sh + e).astype(np.int64))


def test_upcast_every_fp16_scale_every_code():
    sbits = np.arange(1, 0x7C00, dtype=np.uint16)  # every positive finite fp16
    m, e = _f16_parts(sbits)
    for q in range(-7, 8):
        codes = np.full((sbits.size, 64), q, dtype=np.int8)
        got = bf16_to_f64(wo.upcast(codes, sbits[None, :])[0])
        if q == 0:
            want = np.zeros(sbits.size)
        else:
            want = np.sign(q) * _round_int_to_bf16_value(abs(q) * m, e)
        np.testing.assert_array_equal(got, want, err_msg=f"q={q}")


def test_quantize_weights_planted_columns():
    rng = np.random.default_rng(11)
    K, N = 192, 5
    sc = np.array([[0x3C00, 0x2E00, 0x4100, 0x1A00, 0x3500],
                   [0x3800, 0x4400, 0x2C00, 0x3E00, 0x0200],
                   [0x5000, 0x3A00, 0x3C00, 0x0001, 0x4A00]], dtype=np.uint16)  # [K/64][N], at most 3 significant bits
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[:, ::64] = 7  # each group's max |q| is 7, so max|w| / 7 is the group's scale
    s = sc.view(np.float16).astype(np.float64)
    W = q.T.astype(np.float64) * np.repeat(s, 64, axis=0)  # [K][N]: s q has at most 6 significant bits
    Wb = bf16_value_to_bits(W)
    assert np.array_equal(bf16_to_f64(Wb), W), "planted weights must be exact bf16 values"
    codes, sW = wo.quantize_weights(Wb)
    assert codes.shape == (N, K) and sW.shape == (K // 64, N)
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(sW, sc)


def test_forward_triple_loop_and_plain_product():
    rng = np.random.default_rng(12)
    M, K, N = 3, 128, 5
    X = bf16_value_to_bits(rng.standard_normal((M, K)).astype(np.float32).astype(np.float64))
    W = bf16_value_to_bits(rng.standard_normal((K, N)).astype(np.float32).astype(np.float64))
    codes, sW = wo.quantize_weights(W)
    Y = wo.forward(X, codes, sW)
    Wd = bf16_to_f64(wo.upcast(codes, sW))
    Xv = bf16_to_f64(X)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                # weight k of column n: code codes[n][k] times the scale of group k // 64
                sv = float(np.array([sW[k // 64, n]], dtype=np.uint16).view(np.float16)[0])
                w = float(Wd[k, n])
                assert abs(w - sv * codes[n, k]) <= abs(sv * codes[n, k]) * 2.0 ** -8
                acc += float(Xv[m, k]) * w
            ref[m, n] = acc
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    # sub-blocks
    np.testing.assert_allclose(wo.forward(X, codes, sW, rows=[2], cols=[0, 4]), ref[[2]][:, [0, 4]], rtol=1e-12)


def test_forward_reduces_to_plain_product_on_exact_weights():
    """Weights that already are s q with bf16-exact products: the quantizer returns them
    unchanged and the layer is the plain product X W."""
    rng = np.random.default_rng(13)
    M, K, N = 4, 256, 6
    q = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    q[:, ::64] = -7
    s = np.ldexp(1.0, rng.integers(-6, 4, size=(K // 64, N)))  # powers of two: s q is exact in bf16
    W = q.T.astype(np.float64) * np.repeat(s, 64, axis=0)
    Wb = bf16_value_to_bits(W)
    X = bf16_value_to_bits(rng.standard_normal((M, K)).astype(np.float32).astype(np.float64))
    codes, sW = wo.quantize_weights(Wb)
    np.testing.assert_array_equal(bf16_to_f64(wo.upcast(codes, sW)), W)
    np.testing.assert_array_equal(wo.forward(X, codes, sW), bf16_to_f64(X) @ W)
