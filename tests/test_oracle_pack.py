"""Pins of the oracle's offline pack (SVD split, residual quantization, LoRA fold).

The SVD split is checked against closed forms that do not reuse the oracle's SVD
call: singular values from the eigenvalues of the Gram matrix (a different LAPACK
routine), the Eckart-Young error, orthonormality, and the rank-0 / exact-low-rank
reductions.  The quality claims of the pages are checked in direction only (the
pages print no numbers for them): the residual R quantizes with less error than the
smoothed weight (jeonghoonpark.com "SVDQuant" review, section 4.2; ch3chohch3.github.io
"从 Smooth Quant 到 SVD Quant", section "量化方案"), and smoothing alone inflates the
weight's quantization error (the review's section 4.2, "After Smoothing").
"""
import numpy as np
import pytest

from oracle import pack, quant, forward
from oracle.numerics import bf16_to_f64
from bit_diffusion_model_amd.workloads import make, random_layer


def _svd_pack(wl, rank=None):
    a = quant.channel_absmax_cols(wl.calib)
    return pack.pack_weights(wl.W, a, wl.alpha, wl.rank if rank is None else rank, wl.fmt)


@pytest.fixture(scope="module")
def c0():
    wl = make("C0")
    return wl, _svd_pack(wl)


def test_singular_values_match_gram_eigenvalues(c0):
    wl, p = c0
    Wh = p["W_hat"]
    lam = np.linalg.eigvalsh(Wh @ Wh.T)[::-1]  # symmetric eigensolver, not an SVD
    np.testing.assert_allclose(p["sigma"] ** 2, np.maximum(lam, 0), rtol=1e-9, atol=1e-9 * lam[0])


def test_eckart_young_and_orthonormality(c0):
    wl, p = c0
    r = wl.rank
    Wh, L1, L2, S = p["W_hat"], p["L1"], p["L2"], p["sigma"]
    lam = np.sort(np.linalg.eigvalsh(Wh.T @ Wh))[::-1]
    err2 = np.sum((Wh - L1 @ L2) ** 2)
    np.testing.assert_allclose(err2, lam[r:].sum(), rtol=1e-9)
    np.testing.assert_allclose(np.sum((L1 @ L2) ** 2), lam[:r].sum(), rtol=1e-9)
    np.testing.assert_allclose(L2 @ L2.T, np.eye(r), atol=1e-12)
    np.testing.assert_allclose(L1.T @ L1, np.diag(S[:r] ** 2), atol=1e-9 * S[0] ** 2)
    # the kept directions are the largest: any rank-r subset of others is worse
    assert np.all(np.diff(S) <= 0)


def test_reconstruction_with_stored_bf16_factors(c0):
    wl, p = c0
    rec = p["L1b"] @ p["L2b"] + p["R"]
    assert np.abs(rec - p["W_hat"]).max() <= 1e-12 * np.abs(p["W_hat"]).max()
    # the stored factors are bf16 values: widening their bit patterns gives them back
    assert np.array_equal(bf16_to_f64(p["L1_bits"]), p["L1b"])
    assert np.array_equal(bf16_to_f64(p["L2_bits"]), p["L2b"])
    # rounding the factors to bf16 moves L1 L2 by at most bf16 precision
    d = np.abs(p["L1b"] @ p["L2b"] - p["L1"] @ p["L2"]).max()
    assert d <= 2 ** -7 * np.abs(p["L1"] @ p["L2"]).max()


def test_rank0_is_plain_smoothed_quantization(c0):
    wl, _ = c0
    p0 = _svd_pack(wl, rank=0)
    assert p0["L1b"].shape == (wl.K, 0) and p0["L2b"].shape == (0, wl.N)
    assert np.array_equal(p0["R"], p0["W_hat"])
    codes, sc = quant.quantize_int4(p0["W_hat"].astype(np.float32).T)
    assert np.array_equal(p0["codesW"], codes) and np.array_equal(p0["sW"], sc.T)


def test_exact_low_rank_weight_leaves_tiny_residual():
    rng = np.random.default_rng(21)
    K, N, r = 128, 96, 4
    from bit_diffusion_model_amd.workloads import bf16_bits_from_f64
    Wb = bf16_bits_from_f64(rng.standard_normal((K, r)) @ rng.standard_normal((r, N)))
    # bf16 rounding of W itself breaks exact low rank only at the 2^-9 level
    p = pack.pack_weights(Wb, None, 0.5, r, "int4")
    assert np.abs(p["R"]).max() <= 2 ** -6 * np.abs(p["W_hat"]).max()
    p_more = pack.pack_weights(Wb, None, 0.5, r + 4, "int4")
    assert np.abs(p_more["R"]).max() <= 2 ** -6 * np.abs(p["W_hat"]).max()


def test_residual_layout_and_scales(c0):
    """codesW [N][K] are the per-output-column INT4 codes of R32 along K; sW is [K/64][N]."""
    wl, p = c0
    R32 = p["R32"]
    n, g = 17, 2
    col = R32[g * 64:(g + 1) * 64, n]
    codes, sb = quant.quantize_int4(col[None, :])
    assert np.array_equal(p["codesW"][n, g * 64:(g + 1) * 64], codes[0])
    assert p["sW"][g, n] == sb[0, 0]
    assert p["qW"].shape == (wl.N, wl.K // 2)


def test_residual_quantizes_better_than_smoothed_weight():
    for name in ["C0"]:
        wl = make(name)
        p = _svd_pack(wl)
        err_R = np.linalg.norm(p["R32"].T - quant.dequant_int4(p["codesW"], p["sW"].T))
        W_hat32 = p["W_hat"].astype(np.float32).T
        cW, sW = quant.quantize_int4(W_hat32)
        err_W = np.linalg.norm(W_hat32 - quant.dequant_int4(cW, sW))
        assert err_R < 0.8 * err_W, (err_R, err_W)


def test_svdquant_beats_smoothing_only_and_naive_w4a4():
    """End-to-end error |XW - Y| for naive W4A4, smoothing-only W4A4, and SVDQuant."""
    wl = make("C0")
    X = bf16_to_f64(wl.X)
    W = bf16_to_f64(wl.W)
    ref = X @ W
    a = quant.channel_absmax_cols(wl.X)
    errs = {}
    for label, act, rank in [("naive", None, 0), ("smooth", a, 0), ("svdquant", a, wl.rank)]:
        p = pack.pack_weights(wl.W, act, wl.alpha, rank, "int4")
        Y = forward.forward(wl.X, p)["Y"]
        errs[label] = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    assert errs["svdquant"] < errs["smooth"] < errs["naive"], errs
    assert errs["svdquant"] < 0.5 * errs["naive"], errs


def test_error_bound_invariant():
    """|XW - Q(X)Q(W)|_F <= |X|_F |W - Q(W)|_F + |X - Q(X)|_F (|W|_F + |W - Q(W)|_F):
    the four factors the review's section 4.1 names, combined by the triangle
    inequality and sub-multiplicativity (the equation itself is missing from the page)."""
    for seed in range(3):
        wl = random_layer(32, 256, 48, 0, 100 + seed, x_out=3, w_out=2)
        X = bf16_to_f64(wl.X).astype(np.float32)
        W = bf16_to_f64(wl.W).astype(np.float32)
        cX, sX = quant.quantize_int4(X)
        QX = quant.dequant_int4(cX, sX)
        cW, sW = quant.quantize_int4(W.T)
        QW = quant.dequant_int4(cW, sW).T
        X64, W64 = X.astype(np.float64), W.astype(np.float64)
        lhs = np.linalg.norm(X64 @ W64 - QX @ QW)
        eW = np.linalg.norm(W64 - QW)
        eX = np.linalg.norm(X64 - QX)
        rhs = np.linalg.norm(X64) * eW + eX * (np.linalg.norm(W64) + eW)
        assert lhs <= rhs


def test_lora_fold_keeps_residual_and_adds_adapter():
    wl = random_layer(24, 256, 64, 8, 77, lora_rank=4)
    a = quant.channel_absmax_cols(wl.X)
    p = pack.pack_weights(wl.W, a, wl.alpha, wl.rank, "int4")
    pl = pack.fold_lora(p, wl.lora_A, wl.lora_B)
    assert pl["rank"] == 12
    assert np.array_equal(pl["qW"], p["qW"]) and np.array_equal(pl["sW"], p["sW"])
    y0 = forward.forward(wl.X, p)["Y"]
    y1 = forward.forward(wl.X, pl)["Y"]
    X = bf16_to_f64(wl.X)
    xab = X @ bf16_to_f64(wl.lora_A) @ bf16_to_f64(wl.lora_B)
    # difference equals X A B up to bf16 rounding of the folded factor and fp32 X_hat
    assert np.abs((y1 - y0) - xab).max() <= 2 ** -7 * np.abs(xab).max() + 1e-9
