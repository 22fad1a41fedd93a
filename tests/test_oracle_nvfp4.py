"""Pins of the oracle's NVFP4-style group-16 quantizer (E2M1 codes, E4M3 group scales,
an fp32 tensor scale), the variant the ch3chohch3.github.io post discusses in its
section "个人见解".

* hand-derived cases (tests/golden/nvfp4_cases.json): E4M3 rounding at ties, binade and
  subnormal boundaries and saturation; the tensor scale; whole groups whose quotients
  hit E2M1 ties, with a subnormal, a saturated and a vanishing group scale;
* E4M3 rounding against an exhaustive nearest search over all 127 finite non-negative
  E4M3 values (ties to the even code), on values across the whole range;
* invariants: codes on the E2M1 grid, |t| <= 6, the group max mapping to 6 whenever its
  scale is a normal unsaturated E4M3 value, the dequantization error bound;
* the forward against a brute-force triple loop;
* the direction of the post's claim: under this format SVDQuant's relative error is below
  bare NVFP4's on an outlier workload (the post measures 1.16-3x; direction only).
"""
import json
import os

import numpy as np
import pytest

from bit_diffusion_model_amd.workloads import random_layer
from oracle import forward, pack, quant

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "nvfp4_cases.json")))


def test_e4m3_hand_derived():
    for c in GOLD["e4m3"]:
        x, want = float.fromhex(c["x"]), float.fromhex(c["v"])
        assert quant.e4m3_round(np.array([x]))[0] == want, c["why"]


def test_tensor_scale_hand_derived():
    for c in GOLD["tensor_scale"]:
        assert quant.nvfp4_tensor_scale(float.fromhex(c["amax"])) == np.float32(float.fromhex(c["S"])), c["why"]


def test_group_quantization_hand_derived():
    for c in GOLD["groups"]:
        v = np.array([float.fromhex(x) for x in c["v"]], np.float32)[None, :]
        codes, e = quant.quantize_nvfp4(v, np.float32(float.fromhex(c["S"])))
        assert e[0, 0] == c["e4m3"], c["why"]
        np.testing.assert_array_equal(codes[0], np.array(c["codes"], np.uint8), err_msg=c["why"])


def test_e4m3_exhaustive_nearest():
    table = quant.e4m3_value(np.arange(127, dtype=np.uint8))  # every finite non-negative value
    rng = np.random.default_rng(1)
    x = np.concatenate([table, (table[1:] + table[:-1]) / 2,  # every value and every tie
                        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 20000))])
    got = quant.e4m3_round(x)
    for xi, gi in zip(x, got):
        if xi >= 448:
            assert gi == 448
            continue
        d = np.abs(table - xi)
        cand = np.flatnonzero(d == d.min())
        best = cand[0] if len(cand) == 1 else [c for c in cand if c % 2 == 0][0]  # ties: even code
        assert gi == table[best], (xi, gi, table[best])
    np.testing.assert_array_equal(quant.e4m3_bits(table), np.arange(127, dtype=np.uint8))


def test_invariants_and_error_bound():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-3, 2, (64, 1))).astype(np.float32)
    S = quant.nvfp4_tensor_scale(np.abs(v).max())
    codes, e = quant.quantize_nvfp4(v, S)
    s = quant.e4m3_value(e)
    sigma = (s.astype(np.float32) * S).astype(np.float32)
    g = v.reshape(64, -1, 16)
    vals = quant.e2m1_value(codes).reshape(64, -1, 16)
    assert set(np.unique(codes & 7)) <= set(range(8))
    # the group max maps to +-6 when its scale is normal and not saturated
    normal = (s >= 2.0 ** -6) & (s < 448)
    amax_idx = np.abs(g).argmax(axis=-1)
    top = np.take_along_axis(np.abs(vals), amax_idx[..., None], axis=-1)[..., 0]
    assert (top[normal] == 6).all()
    # |v - S s e2m1| <= half the local grid gap (at most sigma) plus, where |v| / sigma
    # exceeds 6 (a subnormal or saturated group scale rounded down), the excess over 6 sigma
    deq = quant.dequant_nvfp4(codes, e, S).reshape(g.shape)
    sg = sigma[..., None].astype(np.float64)
    bound = sg * (1 + 1e-6) + np.maximum(0.0, np.abs(g) - 6 * sg)
    assert (np.abs(deq - g) <= bound + 1e-30).all()


def _brute(wl, p):
    """Y[m][n] = S_X S_W sum_k sX sW vX vW + (X_hat L1) L2 by element loops over groups of 16."""
    Xh = quant.smooth_activations(wl.X, p["inv_s32"])
    M, K = Xh.shape
    N = wl.N
    dX = np.zeros((M, K))
    for m in range(M):
        c, e = quant.quantize_nvfp4(Xh[m:m + 1], p["S_X"])
        for k in range(K):
            dX[m, k] = float(quant.e2m1_value(c[0, k])) * float(quant.e4m3_value(e[0, k // 16])) * float(p["S_X"])
    dW = np.zeros((K, N))
    for n in range(N):
        for k in range(K):
            dW[k, n] = (float(quant.e2m1_value(p["codesW"][n, k])) * float(quant.e4m3_value(p["sW"][k // 16, n]))
                        * float(p["S_W"]))
    Y = dX @ dW
    if p["rank"]:
        Y = Y + (Xh.astype(np.float64) @ p["L1b"]) @ p["L2b"]
    return Y


@pytest.mark.parametrize("M,K,N,r", [(3, 128, 5, 2), (5, 256, 7, 8)])
def test_forward_brute_force(M, K, N, r):
    wl = random_layer(M, K, N, r, 900 + M + N, fmt="nvfp4", x_out=2, w_out=1)
    p = pack.pack_weights(wl.W, quant.channel_absmax_cols(wl.X), wl.alpha, r, "nvfp4")
    Y = forward.forward(wl.X, p)["Y"]
    Yb = _brute(wl, p)
    assert np.abs(Y - Yb).max() <= 1e-12 * np.abs(Yb).max()


def test_svdquant_beats_bare_nvfp4_direction():
    """Relative output error of SVDQuant (smoothing + rank-32 split + NVFP4 residual) and of
    bare NVFP4 (no smoothing, no split) against the exact XW on an outlier workload."""
    wl = random_layer(256, 512, 384, 32, 77, fmt="nvfp4", x_out=5, x_factor=30.0, w_out=4, w_factor=20.0)
    X = quant.smooth_activations(wl.X, np.ones(wl.K, np.float32)).astype(np.float64)
    from oracle.numerics import bf16_to_f64
    ref = X @ bf16_to_f64(wl.W)
    sv = pack.pack_weights(wl.W, quant.channel_absmax_cols(wl.X), 0.5, 32, "nvfp4")
    e_svd = np.linalg.norm(forward.forward(wl.X, sv)["Y"] - ref)
    bare = pack.pack_weights(wl.W, None, 0.5, 0, "nvfp4")
    bare["S_X"] = quant.nvfp4_tensor_scale(np.abs(X).max())  # the same calibration statistic, unsmoothed
    e_bare = np.linalg.norm(forward.forward(wl.X, bare)["Y"] - ref)
    print(f"relative error: SVDQuant {e_svd / np.linalg.norm(ref):.4f}, bare NVFP4 {e_bare / np.linalg.norm(ref):.4f}, "
          f"gain {e_bare / e_svd:.2f}x")
    assert e_svd < e_bare
    # smoothing without the split (rank 0) sits in between on this workload
    sm = pack.pack_weights(wl.W, quant.channel_absmax_cols(wl.X), 0.5, 0, "nvfp4")
    e_sm = np.linalg.norm(forward.forward(wl.X, sm)["Y"] - ref)
    print(f"smoothing only {e_sm / np.linalg.norm(ref):.4f}")
    assert e_svd < e_sm
