"""GPU parity at the full FLUX.1 layer sizes, in the launch configuration bench.py times.

For every named workload (QKV, MLP fc1, MLP fc2, the MXFP4 variant of QKV, QKV at batch
2 with a folded rank-16 LoRA) the HIP path runs on the full input and is compared with
the oracle:
* kernel 1: codes and scales bit-exact for every token, lora_act within its error
  budget for every token;
* kernel 2 (INT4): exact integer group sums on an interior window and on the ragged
  last tiles;
* the layer output: sampled rows x columns (the oracle computes them one by one),
  max |err| <= 2e-2 x RMS of the sampled reference; the unfused baseline's output to
  the same bar and within 1e-5 x RMS of the fused output everywhere.
The pack artifacts come from the oracle's own pack (LAPACK SVD), so no oracle input
comes from the HIP path.  The three workloads that share the QKV weight share one
oracle SVD.
"""
import numpy as np
import pytest

from gpu_helpers import TOL_Y, layer_from_oracle, log, lora_bound, oracle_k1, rel_err, to_dev_bf16

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import make
from oracle import forward as oforward, pack as opack, quant as oquant

pytestmark = pytest.mark.gpu

_svd_cache = {}


def _pack_for(wl):
    """Oracle pack for a workload; the SVD split of a given (W, calibration) is shared."""
    key = (wl.seed if wl.name != "C4" else 1001, wl.name in ("C1", "C3", "C4"), wl.K, wl.N)
    if key not in _svd_cache:
        a = oquant.channel_absmax_cols(wl.calib)
        w = oquant.channel_absmax_rows(wl.W)
        s64, s32, inv = oquant.smoothing_factors(a, w, wl.alpha)
        sp = opack.svd_split(opack.smoothed_weight(wl.W, s32), wl.rank)
        _svd_cache[key] = (s64, s32, inv, sp)
    s64, s32, inv, sp = _svd_cache[key]
    R32 = sp["R"].astype(np.float32)
    codesW, sW = opack.quantize_residual(R32, wl.fmt)
    p = dict(fmt=wl.fmt, K=wl.K, N=wl.N, rank=wl.rank, s64=s64, s32=s32, inv_s32=inv,
             L1b=sp["L1b"], L2b=sp["L2b"], L1_bits=None, L2_bits=None,
             codesW=codesW, qW=opack.pack_codes(codesW, wl.fmt), sW=sW)
    from oracle.numerics import bf16_value_to_bits
    p["L1_bits"] = bf16_value_to_bits(p["L1b"])
    p["L2_bits"] = bf16_value_to_bits(p["L2b"])
    if wl.lora_A is not None:
        p = opack.fold_lora(p, wl.lora_A, wl.lora_B)
    return p


@pytest.mark.parametrize("name", ["C1", "C2a", "C2b", "C3", "C4"])
def test_full_size_layer(name):
    import torch

    wl = make(name)
    log(f"full-size {name}: M={wl.M} K={wl.K} N={wl.N} rank={wl.total_rank} {wl.fmt}")
    p = _pack_for(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    qX, sX, la = lay.quantize_act(X)
    torch.cuda.synchronize()
    log("  kernel 1 done; oracle kernel 1")
    Xh, codes, sc, qX_ref, sX_ref, la_ref = oracle_k1(wl.X, p)
    np.testing.assert_array_equal(qX.cpu().numpy(), qX_ref)
    np.testing.assert_array_equal(sX.cpu().numpy().view(sX_ref.dtype), sX_ref)
    r = p["rank"]
    la_g = la.cpu().numpy().astype(np.float64)
    assert not la_g[:, r:].any()
    assert np.all(np.abs(la_g[:, :r] - la_ref) <= lora_bound(Xh, p["L1b"]))
    log("  kernel 1 bit-exact; forward")
    Y = lay.forward(X)  # the public entry point, same launch as bench.py
    if wl.fmt == "int4":
        M, N = wl.M, wl.N
        wins = [(M // 2 - 70, N // 2 - 90, 140, 180), (M - 77, N - 61, 77, 61)]
        for m0, n0, mt, nt in wins:
            I = lay.group_sums(qX, m0, n0, mt, nt).cpu().numpy()
            I_ref = oforward.group_sums(codes[m0:m0 + mt], p["codesW"][n0:n0 + nt], 64)
            np.testing.assert_array_equal(I, I_ref)
        log("  group sums exact")
    rng = np.random.default_rng(7)
    # random rows and columns, plus some from the last tile row and column (the tiles
    # kernel 2 may split along K)
    rows = np.unique(np.concatenate([rng.choice(wl.M, 48, replace=False), [0, wl.M - 1],
                                     rng.choice(np.arange((wl.M - 1) // 128 * 128, wl.M), 8)]))
    cols = np.unique(np.concatenate([rng.choice(wl.N, 48, replace=False), [0, wl.N - 1],
                                     rng.choice(np.arange(wl.N // 2, wl.N), 8)]))
    Yg = Y.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64)
    out = oforward.forward(wl.X, p, rows=rows, cols=cols)
    e = rel_err(Yg, out["Y"])
    log(f"  sampled output max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    # the unfused baseline at full size: the same bar, and the fused output up to the
    # order of the two fp32 terms, on every element
    Yu = lay.forward(X, fused=False)
    eu = rel_err(Yu.cpu().numpy()[np.ix_(rows, cols)].astype(np.float64), out["Y"])
    d = float((Yu - Y).abs().max()) / float(Y.double().pow(2).mean().sqrt())
    log(f"  unfused baseline: sampled max|err|/RMS = {eu:.3e}, max|Y_unfused - Y|/RMS = {d:.3e}")
    assert eu <= TOL_Y and d <= 1e-5
