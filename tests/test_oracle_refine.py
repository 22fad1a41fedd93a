"""Pins of the oracle's iterative refinement of the split (oracle.pack.refine_split),
against facts that do not come from the refinement code itself: the plain split it
starts from, the exact decomposition W_hat = L1b L2b + R, Eckart-Young for every
iterate's rank-r split (singular values from a symmetric eigensolver, not the SVD the
oracle calls), and the error of the kept pack recomputed from its stored codes and
scales by the quantizer's own dequantization.
"""
import numpy as np
import pytest

from bit_diffusion_model_amd.workloads import random_layer
from oracle import pack, quant


def _layer(fmt, seed=3, K=256, N=96):
    wl = random_layer(64, K, N, 8, seed, fmt=fmt, x_out=3, w_out=2)
    a = quant.channel_absmax_cols(wl.calib)
    w_absmax = quant.channel_absmax_rows(wl.W)
    _, s32, _ = quant.smoothing_factors(a, w_absmax, wl.alpha)
    return wl, a, pack.smoothed_weight(wl.W, s32)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_iterate_zero_is_the_plain_split(fmt):
    wl, a, W_hat = _layer(fmt)
    best, errors, t = pack.refine_split(W_hat, 8, fmt, 0)
    plain = pack.pack_weights(wl.W, a, wl.alpha, 8, fmt)
    assert t == 0 and len(errors) == 1
    np.testing.assert_array_equal(best["L1b"], plain["L1b"])
    np.testing.assert_array_equal(best["L2b"], plain["L2b"])
    np.testing.assert_array_equal(best["codes"], plain["codesW"])
    np.testing.assert_array_equal(best["sW"], plain["sW"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_kept_pack_error_decomposition_and_monotone_best(fmt):
    wl, a, W_hat = _layer(fmt)
    p = pack.pack_weights(wl.W, a, wl.alpha, 8, fmt, refine_iters=4)
    errors = p["errors"]
    assert len(errors) == 5 and p["best_iter"] == int(np.argmin(errors))
    # exact decomposition with the stored factors
    assert np.array_equal(p["W_hat"], p["L1b"] @ p["L2b"] + p["R"]) or \
        np.abs(p["W_hat"] - (p["L1b"] @ p["L2b"] + p["R"])).max() <= 1e-12 * np.abs(p["W_hat"]).max()
    # the error of the kept pack, from its stored codes and scales
    sc = np.ascontiguousarray(p["sW"].T)
    D = (quant.dequant_int4(p["codesW"], sc) if fmt == "int4" else quant.dequant_mxfp4(p["codesW"], sc)).T
    E = np.linalg.norm(p["W_hat"] - p["L1b"] @ p["L2b"] - D)
    assert E == pytest.approx(min(errors), rel=1e-12)
    # more iterations: the same first iterates (deterministic), never a worse pack
    _, e2, _ = pack.refine_split(p["W_hat"], 8, fmt, 2)
    assert e2 == errors[:3]
    assert min(errors) <= min(e2) <= errors[0]
    # on this layer refinement does lower the error (the page's claim)
    assert min(errors) < errors[0]


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_every_iterate_is_a_best_rank_r_split_of_its_target(fmt):
    _, _, W_hat = _layer(fmt, seed=9, K=128, N=160)
    r = 8
    best, errors, _ = pack.refine_split(W_hat, r, fmt, 3, keep_iterates=True)
    its = best["iterates"]
    assert len(its) == 4
    for t, it in enumerate(its):
        T = it["target"]
        lam = np.sort(np.linalg.eigvalsh(T @ T.T))[::-1]  # symmetric eigensolver
        tail = float(np.clip(lam[r:], 0, None).sum())
        res = np.linalg.norm(T - it["L1"] @ it["L2"]) ** 2
        assert res == pytest.approx(tail, rel=1e-8, abs=1e-10 * lam[0])
        np.testing.assert_allclose(it["L2"] @ it["L2"].T, np.eye(r), atol=1e-10)  # orthonormal rows
        if t:
            # the target is W_hat minus the previous iterate's dequantized residual
            prev = its[t - 1]
            ev = pack.split_error(W_hat, prev["L1b"], prev["L2b"], fmt)
            np.testing.assert_array_equal(T, W_hat - ev["D"])
        assert it["err"] == errors[t]
