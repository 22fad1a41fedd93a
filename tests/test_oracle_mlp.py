"""Pins of the oracle's chained MLP pair (GELU between two layer forwards).

* GELU against standard normal CDF values from printed tables and quantiles
  (Phi(1), Phi(2), Phi(3), the 0.95 / 0.975 / 0.995 quantiles) and the far negative tail
  (Q(10) = 7.6198530241605e-24), so a missing 1/sqrt(2), a wrong sign of the erfc
  argument or a lost factor 1/2 fails;
* the identity GELU(x) - GELU(-x) = x;
* the composition on tiny layers against an independent evaluation: GELU by
  scipy.stats.norm.cdf (another routine than the oracle's erfc), bf16 rounding by a
  brute-force nearest-of-neighbours search, then the (separately pinned) layer forward;
  a GELU applied to the wrong tensor, a missing or doubled rounding or a swapped layer
  order changes the result.
"""
import numpy as np
import pytest
from scipy.stats import norm

from oracle import forward, pack, quant
from bit_diffusion_model_amd.workloads import random_layer


@pytest.mark.parametrize("x,phi", [
    (0.0, 0.5),
    (1.0, 0.8413447460685429),
    (2.0, 0.9772498680518208),
    (3.0, 0.9986501019683699),
    (-1.0, 0.15865525393145707),
    (1.6448536269514722, 0.95),
    (1.959963984540054, 0.975),
    (2.5758293035489004, 0.995),
])
def test_gelu_table_values(x, phi):
    g = forward.gelu_erf(np.array([x]))[0]
    assert g == pytest.approx(x * phi, rel=1e-14, abs=1e-300)


def test_gelu_negative_tail_keeps_relative_accuracy():
    # Q(10) = P(Z > 10) = 7.6198530241605e-24 (standard normal tail tables)
    g = forward.gelu_erf(np.array([-10.0]))[0]
    assert g == pytest.approx(-10.0 * 7.6198530241605e-24, rel=1e-12)


def test_gelu_odd_part_identity():
    x = np.random.default_rng(5).standard_normal(10000) * 4
    d = forward.gelu_erf(x) - forward.gelu_erf(-x)
    np.testing.assert_allclose(d, x, rtol=1e-14, atol=1e-15)


def _bf16_nearest_brute(v):
    """Nearest bf16 (ties to the even pattern) by comparing two neighbours in fp64: the
    bf16 patterns t and t + 1 with t the top half of fp32(v).  If the fp32 step crosses a
    bf16 value, v sits within an fp32 half-step of pattern t, which is then the nearest."""
    out = np.empty(v.shape, dtype=np.uint16)
    flat, o = v.ravel(), out.ravel()
    for i, x in enumerate(flat):
        if x == 0.0:
            o[i] = 0x8000 if np.signbit(x) else 0
            continue
        t = int(np.array([np.float32(x)]).view(np.uint32)[0] >> 16)
        cands = [t, t + 1]
        vals = [float(np.array([c << 16], dtype=np.uint32).view(np.float32)[0]) for c in cands]
        d = [abs(vv - x) for vv in vals]
        if d[0] != d[1]:
            o[i] = cands[0] if d[0] < d[1] else cands[1]
        else:
            o[i] = cands[0] if cands[0] % 2 == 0 else cands[1]
    return out


def _pair(M, K1, N1, N2, r1, r2, seed):
    l1 = random_layer(M, K1, N1, r1, seed)
    p1 = pack.pack_weights(l1.W, quant.channel_absmax_cols(l1.X), l1.alpha, r1, "int4")
    # fc2's calibration: its input as the pair produces it
    G_cal = forward.mlp_hidden(l1.X, p1)["G_bits"]
    l2 = random_layer(M, N1, N2, r2, seed + 1)
    p2 = pack.pack_weights(l2.W, quant.channel_absmax_cols(G_cal), l2.alpha, r2, "int4")
    return l1, p1, p2


@pytest.mark.parametrize("shape", [(5, 128, 128, 7, 4, 3), (33, 256, 384, 40, 8, 16)])
def test_mlp_composition_against_independent_steps(shape):
    M, K1, N1, N2, r1, r2 = shape
    l1, p1, p2 = _pair(M, K1, N1, N2, r1, r2, seed=77 + M)
    out = forward.mlp_forward(l1.X, p1, p2)
    # independent: fc1 forward (pinned on its own), GELU by the normal CDF routine,
    # brute-force bf16 rounding, fc2 forward
    H = forward.forward(l1.X, p1)["Y"]
    G = H * norm.cdf(H)
    G_bits = _bf16_nearest_brute(G)
    np.testing.assert_array_equal(out["G_bits"], G_bits)
    Y = forward.forward(G_bits, p2)["Y"]
    np.testing.assert_array_equal(out["fc2"]["Y"], Y)
    # a subset of tokens gives those tokens' outputs
    rows = np.array([0, M - 1])
    sub = forward.mlp_forward(l1.X[rows], p1, p2, cols=np.arange(min(5, N2)))
    np.testing.assert_allclose(sub["fc2"]["Y"], Y[rows][:, :min(5, N2)], rtol=1e-12, atol=1e-9)
