"""GPU parity on planted edge cases of the two quantizers.

The quantizer is the review's section 3 equation (Q_X = round(X / s_X), s_X = max|X| /
q_max) with the readings the oracle states: INT4 rounds the exact quotient half to even
with an fp16 scale that saturates at 65504 and an all-zero code group for a zero scale;
FP4 takes the smallest power-of-two scale with 6 * 2^e >= max|X| (E8M0, clamped to
[-127, 127]) and rounds half to even on the E2M1 grid keeping the sign bit.  Random
Gaussian inputs almost never reach these cases, so each group of X here is built to hit
one of them (the smoothing factor is 1, so X_hat = X exactly), and every generator
checks on the oracle side that the case really occurs.  Kernel 1's codes and scales
(both activation forms) must be bit-exact; the forward must match the oracle per case
to the usual 2e-2 x RMS bar, every output written.
"""
import numpy as np
import pytest

from gpu_helpers import (TOL_Y, assert_finite, decode_mma, forward_sentinel, layer_from_oracle, log, oracle_k1,
                         rel_err, sentinel_act, to_dev_bf16)

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import bf16_bits_from_f64, bf16_bits_to_f32
from oracle import forward as oforward, pack as opack, quant as oquant
from oracle.numerics import bf16_value_to_bits, round_f64_to_bf16

pytestmark = pytest.mark.gpu


def _exact_bf16(v):
    """bf16 bits of values that must be bf16-representable (asserted)."""
    v = np.asarray(v, dtype=np.float64)
    b = bf16_bits_from_f64(v)
    assert np.array_equal(bf16_bits_to_f32(b).astype(np.float64), v), "planted value not representable in bf16"
    return b


def _int4_groups(rng):
    """(name, 64 bf16 bits, check_forward) for each INT4 case."""
    G = 64
    out = []

    def ties(s):
        a = 7 * s
        half = (np.arange(7) + 0.5) * s  # x / s = k + 1/2 exactly
        v = rng.choice(np.concatenate([half, -half]), G)
        v[0], v[1] = a, -a
        return v

    out.append(("ties_s1", _exact_bf16(ties(1.0)), True))
    out.append(("ties_s0.75", _exact_bf16(ties(0.75)), True))
    out.append(("ties_s0.625", _exact_bf16(ties(0.625)), True))
    near = np.array([2.5 + 2 ** -6, 2.5 - 2 ** -6, 0.5 + 2 ** -8, 0.5 - 2 ** -9, 6.5 + 2 ** -5, 6.5 - 2 ** -5,
                     3.5 + 2 ** -6, 1.5 - 2 ** -7])
    v = rng.choice(np.concatenate([near, -near]), G)
    v[0] = 7.0
    out.append(("near_ties_s1", _exact_bf16(v), True))
    out.append(("zero", _exact_bf16(np.zeros(G)), True))
    out.append(("neg_zero", np.full(G, 0x8000, np.uint16), True))
    # fp16-subnormal scale coarse enough that the absmax element's quotient rounds to 8:
    # the clamp to 7 acts
    a = 1.484375 * 2.0 ** -20
    v = rng.uniform(-a, a, G)
    v[0] = a
    out.append(("fp16_subnormal_scale_clamped", bf16_bits_from_f64(v), True))
    v = rng.uniform(-1e-4, 1e-4, G)
    v[0] = 1e-4
    out.append(("fp16_subnormal_scale", bf16_bits_from_f64(v), True))
    v = rng.uniform(-1e-9, 1e-9, G)
    out.append(("scale_underflows_to_zero", bf16_bits_from_f64(v), True))
    v = rng.uniform(-1e6, 1e6, G)
    v[0] = 1e6
    out.append(("scale_saturates", bf16_bits_from_f64(v), True))
    v = rng.standard_normal(G)
    v[:32] = rng.uniform(-1e-39, 1e-39, 32)  # bf16 (fp32) denormals next to normal values
    out.append(("fp32_denormals", bf16_bits_from_f64(v), True))
    out.append(("gaussian", bf16_bits_from_f64(rng.standard_normal(G)), True))
    return out


def _fp4_groups(rng):
    G = 32
    out = []
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
    v = rng.choice(np.concatenate([ties, -ties]), G)
    v[0] = 6.0
    out.append(("grid_ties_e0", _exact_bf16(v), True))
    v = rng.uniform(-0.24, 0.0, G)
    v[0] = 6.0
    v[1] = -0.25  # a tie to -0
    out.append(("negative_to_minus_zero", bf16_bits_from_f64(v), True))
    out.append(("zero", _exact_bf16(np.zeros(G)), True))
    out.append(("neg_zero", np.full(G, 0x8000, np.uint16), True))
    v = rng.uniform(-2.0 ** -126, 2.0 ** -126, G)
    v[0] = 2.0 ** -126  # e would be -128: clamped to -127
    out.append(("e8m0_clamp_min_normal", bf16_bits_from_f64(v), True))
    v = rng.uniform(-2.0 ** -130, 2.0 ** -130, G)
    v[0] = 2.0 ** -130
    v[1] = -2.0 ** -130
    out.append(("e8m0_clamp_denormal", bf16_bits_from_f64(v), True))
    v = rng.uniform(-1.5, 1.5, G)
    v[0] = 1.5  # 6 * 2^-2 = 1.5 exactly
    out.append(("exponent_boundary", _exact_bf16(np.where(np.arange(G) == 0, 1.5, round_f64_to_bf16(v))), True))
    v = rng.uniform(-1.5, 1.5, G)
    v[0] = 1.5 + 2 ** -7  # just above: one exponent up
    out.append(("exponent_boundary_above", bf16_bits_from_f64(v), True))
    v = rng.uniform(-3e38, 3e38, G)
    v[0] = 3e38
    out.append(("huge", bf16_bits_from_f64(v), False))  # the forward overflows fp32 on these
    out.append(("gaussian", bf16_bits_from_f64(rng.standard_normal(G)), True))
    return out


def _nv_groups(rng):
    """NVFP4 cases (generated in groups of 32, i.e. two 16-groups): the FP4 cases without
    the fp32-range ones (the tensor scale comes from the largest value, so they would zero
    every other group), plus groups whose E4M3 scale is subnormal or rounds to zero."""
    out = [c for c in _fp4_groups(rng) if c[0] not in ("huge", "e8m0_clamp_min_normal", "e8m0_clamp_denormal")]
    v = rng.uniform(-1e-4, 1e-4, 32)
    v[0] = 1e-4
    out.append(("e4m3_subnormal_scale", bf16_bits_from_f64(v), True))
    v = rng.uniform(-1e-7, 1e-7, 32)
    out.append(("e4m3_scale_rounds_to_zero", bf16_bits_from_f64(v), True))
    return out


def _plain_pack(K, N, rank, fmt, seed, S_X=1.0):
    """A layer with smoothing factor 1 (X_hat = X): residual codes and scales from the
    oracle quantizer on a Gaussian R, bf16 low-rank factors."""
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((K, N)).astype(np.float32)
    codesW, sW = opack.quantize_residual(R, fmt)
    L1b = round_f64_to_bf16(0.05 * rng.standard_normal((K, rank)))
    L2b = round_f64_to_bf16(rng.standard_normal((rank, N)))
    p = dict(fmt=fmt, K=K, N=N, rank=rank, inv_s32=np.ones(K, np.float32), L1b=L1b, L2b=L2b,
             L1_bits=bf16_value_to_bits(L1b), L2_bits=bf16_value_to_bits(L2b), codesW=codesW,
             qW=opack.pack_codes(codesW, fmt), sW=sW)
    if fmt == "nvfp4":
        p["S_W"] = opack.residual_tensor_scale(R)
        p["S_X"] = np.float32(S_X)
    return p


def _planted_X(cases, K, G, rows_per_case, rng):
    """Row block c holds case c in every group (a fresh draw of the case per group)."""
    blocks, names, fwd = [], [], []
    for name, _, f in cases:
        names.append(name)
        fwd.append(f)
    M = rows_per_case * len(cases)
    X = np.empty((M, K), np.uint16)
    for c in range(len(cases)):
        for i in range(rows_per_case):
            m = c * rows_per_case + i
            for g in range(K // G):
                X[m, g * G:(g + 1) * G] = cases[c][1] if (i == 0 and g == 0) else _regen(cases[c][0], G, rng)
    return X, names, fwd


_GEN = {}


def _regen(name, G, rng):
    gens = _GEN[G](rng) if name not in _NV_ONLY else _nv_groups(rng)
    for n, bits, _ in gens:
        if n == name:
            return bits
    raise KeyError(name)


_GEN[64] = _int4_groups
_GEN[32] = _fp4_groups
_NV_ONLY = ("e4m3_subnormal_scale", "e4m3_scale_rounds_to_zero")


def _oracle_side_checks(fmt, names, X, rows_per_case):
    """The planted cases occur: ties, clamps, zero / subnormal / saturated scales, -0."""
    Xh = oquant.smooth_activations(X, np.ones(X.shape[1], np.float32))
    rows = {n: slice(i * rows_per_case, (i + 1) * rows_per_case) for i, n in enumerate(names)}
    if fmt == "int4":
        codes, sb = oquant.quantize_int4(Xh)
        s = sb.view(np.float16).astype(np.float64)
        t = Xh.astype(np.float64).reshape(Xh.shape[0], -1, 64) / np.where(s == 0, 1, s)[..., None]
        frac = np.abs(t - np.floor(t))
        assert (frac[rows["ties_s1"]] == 0.5).any() and (frac[rows["ties_s0.75"]] == 0.5).any()
        assert (frac[rows["ties_s0.625"]] == 0.5).any()
        assert (np.abs(t[rows["fp16_subnormal_scale_clamped"]]) >= 7.5).any(), "clamp case not reached"
        sub = s[rows["fp16_subnormal_scale"]]
        assert ((sub > 0) & (sub < 2.0 ** -14)).all()
        assert (s[rows["scale_underflows_to_zero"]] == 0).all()
        assert (s[rows["scale_saturates"]] == 65504.0).all()
        assert not codes[rows["scale_underflows_to_zero"]].any()
        return codes
    if fmt == "nvfp4":
        S = oquant.nvfp4_tensor_scale(np.abs(Xh).max())
        codes, e = oquant.quantize_nvfp4(Xh, S)
        sub = e[rows["e4m3_subnormal_scale"]]
        assert ((sub > 0) & (sub < 8)).any(), "no subnormal E4M3 scale"
        assert (e[rows["e4m3_scale_rounds_to_zero"]] == 0).all()
        assert (codes[rows["neg_zero"]] == 0x8).all() and (codes[rows["zero"]] == 0).all()
        assert (e[rows["grid_ties_e0"]] == 0x7E).any(), "a group at the tensor maximum takes scale 448"
        return codes
    codes, e = oquant.quantize_mxfp4(Xh)
    assert (e[rows["e8m0_clamp_min_normal"]] == 0).all() and (e[rows["e8m0_clamp_denormal"]] == 0).all()
    assert (codes[rows["neg_zero"]] == 0x8).all() and (codes[rows["zero"]] == 0).all()
    assert (codes[rows["negative_to_minus_zero"]] == 0x8).any()
    assert (e[rows["exponent_boundary"]][:, 0] == 127 - 2).all()
    assert (e[rows["exponent_boundary_above"]][:, 0] == 127 - 1).all()
    return codes


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "nvfp4"])
def test_planted_quantizer_edge_cases(fmt):
    import torch

    G = 64 if fmt == "int4" else 32
    K, N, rank, rpc = 256, 96, 16, 3
    rng = np.random.default_rng({"int4": 2024, "mxfp4": 2025, "nvfp4": 2026}[fmt])
    cases = _nv_groups(rng) if fmt == "nvfp4" else _GEN[G](rng)
    X, names, fwd = _planted_X(cases, K, G, rpc, rng)
    M = X.shape[0]
    log(f"edge cases {fmt}: {len(names)} cases x {rpc} rows, K={K}: {', '.join(names)}")
    _oracle_side_checks(fmt, names, X, rpc)
    Xh = oquant.smooth_activations(X, np.ones(K, np.float32))
    p = _plain_pack(K, N, rank, fmt, 31, S_X=oquant.nvfp4_tensor_scale(np.abs(Xh).max()))
    lay = layer_from_oracle(p)
    Xd = to_dev_bf16(X)
    Xh, codes, sc, qX_ref, sX_ref, la_ref = oracle_k1(X, p)
    qX, sX, la = lay.quantize_act(Xd, out=sentinel_act(lay, M, svdq.ACT_PACKED))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qX.cpu().numpy(), qX_ref)
    np.testing.assert_array_equal(sX.cpu().numpy().view(sX_ref.dtype), sX_ref)
    qm, sm, lam = lay.quantize_act(Xd, out=sentinel_act(lay, M, svdq.ACT_MMA), form=svdq.ACT_MMA)
    c_m, s_m = decode_mma(qm, sm, lam, fmt, K, rank, M=M)[:2]
    if fmt == "int4":
        np.testing.assert_array_equal(c_m, codes)
        np.testing.assert_array_equal(s_m, sX_ref.view(np.float16).astype(np.float64))
    else:
        np.testing.assert_array_equal(c_m, qX_ref)
        np.testing.assert_array_equal(s_m, sX_ref)
    log("  codes and scales bit-exact (packed and MMA forms)")
    Y, _ = forward_sentinel(lay, Xd)
    Yg = Y.cpu().numpy().astype(np.float64)
    Yref = oforward.forward(X, p)["Y"]
    keep = np.concatenate([np.arange(i * rpc, (i + 1) * rpc) for i, f in enumerate(fwd) if f])
    assert np.isfinite(Yg[keep]).all()
    rms_all = np.sqrt(np.mean(Yref[keep] ** 2))
    e = np.abs(Yg[keep] - Yref[keep]).max() / rms_all
    log(f"  forward over every case: max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    # each case against its own RMS too, where it is not negligible next to the others
    for i, (n, f) in enumerate(zip(names, fwd)):
        if not f:
            continue
        rs = slice(i * rpc, (i + 1) * rpc)
        if not Yref[rs].any():
            assert not Yg[rs].any(), n
            log(f"  {n}: output exactly zero")
            continue
        rms = np.sqrt(np.mean(Yref[rs] ** 2))
        if rms < 1e-3 * rms_all:
            continue
        e = np.abs(Yg[rs] - Yref[rs]).max() / rms
        log(f"  {n}: forward max|err|/RMS = {e:.3e}")
        assert e <= TOL_Y, n
