"""Pins of the oracle's forward pass.

* brute force: a plain triple loop over (m, n, k) in Python, in a different order
  and with none of the oracle's block structure, on tiny shapes with a ragged mix;
* rank-0 reduction to the textbook dequantized GEMM (np.matmul);
* R = 0 reduction to the exact low-rank product (X_hat L1) L2 (np.matmul);
* FP4 single-scale tiny shapes, where every output is an exact multiple of
  2^(eX + eW) / 4;
* integer group sums bounded by 64 * 49.
"""
import itertools

import numpy as np
import pytest

from oracle import forward, pack, quant
from oracle.numerics import bf16_to_f64
from bit_diffusion_model_amd.workloads import random_layer


def _pack(wl):
    a = quant.channel_absmax_cols(wl.X)
    return pack.pack_weights(wl.W, a, wl.alpha, wl.rank, wl.fmt)


def _brute(wl, p):
    """Triple loop: Y[m][n] = sum_k deqX[m][k] deqW[k][n] + sum_j (sum_k xh[m][k] L1[k][j]) L2[j][n]."""
    Xh = quant.smooth_activations(wl.X, p["inv_s32"]).astype(np.float64)
    G = 64 if wl.fmt == "int4" else 32
    M, K = Xh.shape
    N = wl.N
    # dequantized activations, element by element
    dX = np.zeros((M, K))
    for m in range(M):
        for g in range(K // G):
            grp = Xh[m, g * G:(g + 1) * G].astype(np.float32)
            if wl.fmt == "int4":
                c, s = quant.quantize_int4(grp[None, :])
                sv = float(np.uint16(s[0, 0]).view(np.float16))
                for i in range(G):
                    dX[m, g * G + i] = int(c[0, i]) * sv
            else:
                c, e = quant.quantize_mxfp4(grp[None, :])
                for i in range(G):
                    dX[m, g * G + i] = float(quant.e2m1_value(c[0, i])) * 2.0 ** (int(e[0, 0]) - 127)
    dW = np.zeros((K, N))
    cW, sW = p["codesW"], p["sW"]
    for n in range(N):
        for k in range(K):
            if wl.fmt == "int4":
                dW[k, n] = int(cW[n, k]) * float(np.uint16(sW[k // G, n]).view(np.float16))
            else:
                dW[k, n] = float(quant.e2m1_value(cW[n, k])) * 2.0 ** (int(sW[k // G, n]) - 127)
    L1, L2 = p["L1b"], p["L2b"]
    r = L1.shape[1]
    Y = np.zeros((M, N))
    for m in range(M):
        la = [sum(Xh[m, k] * L1[k, j] for k in range(K)) for j in range(r)]
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += dX[m, k] * dW[k, n]
            for j in range(r):
                acc += la[j] * L2[j, n]
            Y[m, n] = acc
    return Y


@pytest.mark.parametrize("M,K,N,r,fmt", [
    (1, 128, 1, 0, "int4"), (3, 128, 5, 1, "int4"), (2, 256, 16, 8, "int4"),
    (17, 128, 33, 8, "int4"), (3, 128, 5, 2, "mxfp4"), (5, 256, 7, 8, "mxfp4"),
])
def test_forward_brute_force(M, K, N, r, fmt):
    wl = random_layer(M, K, N, r, 500 + M * 7 + N, fmt=fmt, x_out=2, w_out=1)
    p = _pack(wl)
    out = forward.forward(wl.X, p)
    Yb = _brute(wl, p)
    scale = np.abs(Yb).max() + 1e-30
    assert np.abs(out["Y"] - Yb).max() <= 1e-12 * scale


def test_group_sums_brute_force_and_bound():
    rng = np.random.default_rng(3)
    M, N, K = 5, 6, 192
    cX = rng.integers(-7, 8, (M, K)).astype(np.int8)
    cW = rng.integers(-7, 8, (N, K)).astype(np.int8)
    I = forward.group_sums(cX, cW, 64)
    for g, m, n in itertools.product(range(3), range(M), range(N)):
        assert I[g, m, n] == sum(int(cX[m, k]) * int(cW[n, k]) for k in range(64 * g, 64 * g + 64))
    ext = np.full((1, 64), 7, np.int8)
    assert forward.group_sums(ext, -ext, 64)[0, 0, 0] == -64 * 49
    assert np.abs(I).max() <= 64 * 49


def test_code_product_brute_force_and_group_sum_total():
    """code_product = the plain integer product of the codes, by a Python double loop over
    (m, n) with an explicit sum over k, and equal to the group sums added over groups."""
    rng = np.random.default_rng(4)
    M, N, K = 4, 5, 256
    cX = rng.integers(-7, 8, (M, K)).astype(np.int8)
    cW = rng.integers(-7, 8, (N, K)).astype(np.int8)
    P = forward.code_product(cX, cW)
    for m, n in itertools.product(range(M), range(N)):
        assert P[m, n] == sum(int(cX[m, k]) * int(cW[n, k]) for k in range(K))
    np.testing.assert_array_equal(P, forward.group_sums(cX, cW, 64).sum(axis=0))


def test_rank0_reduces_to_dequantized_gemm():
    wl = random_layer(40, 256, 72, 0, 9, x_out=3)
    p = _pack(wl)
    out = forward.forward(wl.X, p)
    DX = quant.dequant_int4(out["codesX"], out["scalesX"])
    DW = quant.dequant_int4(p["codesW"], p["sW"].T)  # [N][K]
    ref = np.matmul(DX, DW.T)
    assert np.abs(out["Y"] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_zero_residual_reduces_to_low_rank_product():
    wl = random_layer(40, 256, 72, 8, 10, x_out=3)
    p = dict(_pack(wl))
    p["codesW"] = np.zeros_like(p["codesW"])
    out = forward.forward(wl.X, p)
    Xh = quant.smooth_activations(wl.X, p["inv_s32"]).astype(np.float64)
    ref = np.matmul(np.matmul(Xh, p["L1b"]), p["L2b"])
    assert np.abs(out["Y"] - ref).max() <= 1e-12 * np.abs(ref).max()


def test_mxfp4_single_scale_outputs_are_exact_grid_multiples():
    rng = np.random.default_rng(4)
    M, N, K = 6, 5, 128
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    cX = rng.integers(0, 16, (M, K)).astype(np.uint8)
    cW = rng.integers(0, 16, (N, K)).astype(np.uint8)
    cX[:, 0] = 7  # each group contains a 6 so the group scale stays put
    eX = np.full((M, K // 32), 127 + 2, np.uint8)
    eW = np.full((K // 32, N), 127 - 3, np.uint8)
    Y = forward.residual_mxfp4(cX, eX, cW, eW)
    v = lambda c: np.where(c & 8, -grid[c & 7], grid[c & 7])
    ref = (v(cX).astype(np.float64) @ v(cW).T.astype(np.float64)) * 2.0 ** (2 - 3)
    assert np.array_equal(Y, ref)
    unit = 2.0 ** (2 - 3) / 4
    assert np.array_equal(np.rint(Y / unit) * unit, Y)


def test_sampled_rows_cols_match_full():
    wl = random_layer(33, 256, 40, 8, 12)
    p = _pack(wl)
    full = forward.forward(wl.X, p)["Y"]
    rows = np.array([0, 5, 32])
    cols = np.array([1, 39, 7])
    sub = forward.forward(wl.X, p, rows=rows, cols=cols)["Y"]
    np.testing.assert_allclose(sub, full[np.ix_(rows, cols)], rtol=1e-13, atol=1e-13)
