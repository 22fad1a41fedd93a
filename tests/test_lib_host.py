"""Host-side tests of libsvdq.so (no GPU needed).

* the library loads and exports every function include/svdq.h declares;
* the residual quantizer and the LoRA fold are bit-exact against the oracle on the
  oracle's own inputs;
* the C++ pack (own Gram + eigensolver SVD) is checked against the oracle's LAPACK pack
  by property: identical smoothing factors, the same rank-r subspace (singular values,
  Eckart-Young error, factor agreement up to sign), R equal to W_hat minus the
  library's own rounded factors, and the library's codes equal to its quantizer on R;
* argument validation returns the documented status codes with a message.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import make, random_layer
from oracle import pack as opack, quant as oquant
from oracle.numerics import bf16_to_f64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_function():
    hdr = open(os.path.join(ROOT, "include", "svdq.h")).read()
    declared = set(re.findall(r"\b(svdq_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations parsed"
    L = svdq.lib()
    for name in sorted(declared):
        assert hasattr(L, name), name
    assert declared == set(svdq.EXPORTS)


def test_act_absmax_matches_oracle():
    wl = make("C0")
    np.testing.assert_array_equal(svdq.act_absmax(wl.X), oquant.channel_absmax_cols(wl.X).astype(np.float32))


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "nvfp4"])
def test_residual_quantizer_bit_exact(fmt):
    rng = np.random.default_rng(8)
    K, N = 256, 96
    R = (rng.standard_normal((K, N)) * 10.0 ** rng.uniform(-3, 2, (1, N))).astype(np.float32)
    R[:, 3] = 0.0
    R[5:70, 7] = np.float32(0.5) * (np.arange(65) % 15 - 7)  # exact ties at s = 1
    R[:64, 8] = (np.arange(64) - 32).astype(np.float32) / 4.0
    R[:64, 9] = np.linspace(-1e-9, 1e-9, 64).astype(np.float32)  # the fp16 scale underflows to 0: codes 0
    R[64:128, 9] = np.float32(1e6) * np.linspace(-1, 1, 64).astype(np.float32)  # the scale saturates
    codes, sc = opack.quantize_residual(R, fmt)
    qW, sW, tw = svdq.quantize_weights(R, svdq.FMT[fmt], with_tscale=True)
    np.testing.assert_array_equal(qW, opack.pack_codes(codes, fmt))
    np.testing.assert_array_equal(sW, sc)
    if fmt == "nvfp4":
        assert np.float32(tw) == opack.residual_tensor_scale(R)


def test_nvfp4_pack_and_device_layout():
    """The library's NVFP4 pack: codes are the oracle quantizer on the library's own R under
    the library's tensor scales (both equal to the oracle's definitions), and the prepared
    device layout decodes back to those codes and scales."""
    wl = random_layer(64, 256, 200, 8, 3, fmt="nvfp4", x_out=3, w_out=2)
    a = svdq.act_absmax(wl.calib)
    hp = svdq.pack_weights(wl.W, a, wl.alpha, 8, svdq.NVFP4_G16, want_R=True)
    codes, sc = opack.quantize_residual(hp.R, "nvfp4")
    np.testing.assert_array_equal(hp.qW, opack.pack_codes(codes, "nvfp4"))
    np.testing.assert_array_equal(hp.sW, sc)
    assert np.float32(hp.tscale_w) == opack.residual_tensor_scale(hp.R)
    assert np.float32(hp.tscale_x) == oquant.nvfp4_tensor_scale((a * hp.inv_s).astype(np.float32).max())
    K, N = 256, 200
    qo, so = svdq.prepare_weights(K, N, svdq.NVFP4_G16, hp.qW, hp.sW)
    # column n's 64-byte stage segment at (n / 2) K + (b / 64) 128 + (n % 2) 64; inside each
    # 64-block code k at nibble 2 (16 ((k / 8) % 2) + 4 (k / 16)) + k % 8
    for n in (0, 1, 7, N - 1):
        row = np.concatenate([qo[(n // 2) * K + (b // 64) * 128 + (n % 2) * 64:][:64] for b in range(0, K // 2, 64)])
        nib = np.stack([row & 15, row >> 4], axis=1).reshape(-1)
        for k0 in range(0, K, 64):
            for k in range(64):
                pos = 2 * (16 * ((k >> 3) & 1) + 4 * (k >> 4)) + (k & 7)
                assert nib[k0 + pos] == codes[n, k0 + k]
    Np = (N + 3) // 4 * 4
    s4 = so.reshape(K // 64, Np, 4)
    np.testing.assert_array_equal(s4[:, :N].transpose(0, 2, 1).reshape(K // 16, N), sc)
    assert not s4[:, N:].any()


@pytest.fixture(scope="module")
def c0_both():
    wl = make("C0")
    a = svdq.act_absmax(wl.X)
    lib = svdq.pack_weights(wl.W, a, wl.alpha, wl.rank, svdq.INT4_G64, want_R=True)
    orc = opack.pack_weights(wl.W, oquant.channel_absmax_cols(wl.X), wl.alpha, wl.rank, "int4")
    return wl, lib, orc


def _factor_checks(lib, orc, r):
    L1l = bf16_to_f64(lib.L1t).T  # [K][r]
    L2l = bf16_to_f64(lib.L2)
    # per component: equal to the oracle's up to a sign (bf16 rounding is sign-symmetric)
    agree = 0
    total = 0
    for t in range(r):
        sgn = np.sign(np.sum(L1l[:, t] * orc["L1b"][:, t]))
        agree += np.sum(L1l[:, t] == sgn * orc["L1b"][:, t]) + np.sum(L2l[t] == sgn * orc["L2b"][t])
        total += L1l.shape[0] + L2l.shape[1]
    return agree / total


def test_pack_smoothing_bit_exact(c0_both):
    wl, lib, orc = c0_both
    np.testing.assert_array_equal(lib.s, orc["s32"])
    np.testing.assert_array_equal(lib.inv_s, orc["inv_s32"])


def test_pack_svd_split_properties(c0_both):
    wl, lib, orc = c0_both
    r = wl.rank
    assert _factor_checks(lib, orc, r) > 0.999
    L1l = bf16_to_f64(lib.L1t).T
    L2l = bf16_to_f64(lib.L2)
    Wh = orc["W_hat"]
    # R is W_hat minus the library's own rounded factors (fp32 storage)
    np.testing.assert_allclose(lib.R, (Wh - L1l @ L2l).astype(np.float32), rtol=0, atol=2e-6 * np.abs(Wh).max())
    # Eckart-Young with the library's factors, up to their bf16 rounding
    lam = np.sort(np.linalg.eigvalsh(Wh @ Wh.T))[::-1]
    err2 = np.sum((Wh - L1l @ L2l) ** 2)
    assert abs(err2 - lam[r:].sum()) <= 2e-3 * lam[:r].sum()
    # rows of L2 orthonormal to bf16 precision
    np.testing.assert_allclose(L2l @ L2l.T, np.eye(r), atol=2e-2)
    # codes are the library's quantizer on its own R
    qW, sW = svdq.quantize_weights(lib.R, svdq.INT4_G64)
    np.testing.assert_array_equal(qW, lib.qW)
    np.testing.assert_array_equal(sW, lib.sW)


@pytest.mark.parametrize("K,N,r,fmt", [(256, 640, 16, "int4"), (640 // 128 * 128 + 128, 200, 12, "mxfp4"),
                                       (384, 384, 0, "int4"), (128, 64, 64, "int4"), (256, 320, 16, "nvfp4"),
                                       (256, 96, 0, "nvfp4")])
def test_pack_matches_oracle_subspace(K, N, r, fmt):
    wl = random_layer(96, K, N, r, 4242 + K + N, fmt=fmt, x_out=3, w_out=2)
    a = svdq.act_absmax(wl.X)
    lib = svdq.pack_weights(wl.W, a, wl.alpha, r, svdq.FMT[fmt], want_R=True)
    orc = opack.pack_weights(wl.W, oquant.channel_absmax_cols(wl.X), wl.alpha, r, fmt)
    np.testing.assert_array_equal(lib.s, orc["s32"])
    if r:
        assert _factor_checks(lib, orc, r) > 0.995
        P_l = bf16_to_f64(lib.L1t).T @ bf16_to_f64(lib.L2)
        P_o = orc["L1b"] @ orc["L2b"]
        assert np.abs(P_l - P_o).max() <= 2 ** -6 * np.abs(P_o).max()
    else:
        np.testing.assert_array_equal(lib.R, orc["R32"])
        np.testing.assert_array_equal(lib.qW, orc["qW"])
        np.testing.assert_array_equal(lib.sW, orc["sW"])


def _lib_split_error(hp, W_bits, fmt):
    """E = ||W_hat - L1 L2 - deq(Q(R))||_F of a library pack, recomputed by the oracle
    from the pack's own s, factors, codes and scales."""
    Wh = opack.smoothed_weight(W_bits, hp.s)
    nib = oquant.unpack_nibbles(hp.qW)
    sc = np.ascontiguousarray(hp.sW.T)
    if fmt == "int4":
        D = oquant.dequant_int4(oquant.nibble_to_int4(nib), sc)
    elif fmt == "nvfp4":
        D = oquant.dequant_nvfp4(nib, sc, hp.tscale_w)
    else:
        D = oquant.dequant_mxfp4(nib, sc)
    P = bf16_to_f64(hp.L1t).T @ bf16_to_f64(hp.L2) if hp.rank else 0.0
    return float(np.linalg.norm(Wh - P - D.T))


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "nvfp4"])
def test_refined_pack(fmt):
    """svdq_pack_weights_refined: iters = 0 is svdq_pack_weights bit for bit; with
    iterations, the errors it reports follow the oracle's refinement, and the kept pack
    attains the smallest of them."""
    wl = random_layer(64, 256, 96, 8, 3, fmt=fmt, x_out=3, w_out=2)
    a = svdq.act_absmax(wl.calib)
    F = svdq.FMT[fmt]
    plain = svdq.pack_weights(wl.W, a, wl.alpha, 8, F, want_R=True)
    r0 = svdq.pack_weights(wl.W, a, wl.alpha, 8, F, want_R=True, refine_iters=1)
    hp = svdq.pack_weights(wl.W, a, wl.alpha, 8, F, want_R=True, refine_iters=4)
    assert r0.errors[0] == hp.errors[0]
    assert r0.errors[0] == pytest.approx(_lib_split_error(plain, wl.W, fmt), rel=1e-9)
    if np.argmin(r0.errors) == 0:
        for f in ("L1t", "L2", "qW", "sW", "R"):
            np.testing.assert_array_equal(getattr(r0, f), getattr(plain, f))
    # the oracle's refinement on the same smoothed weight
    orc = opack.pack_weights(wl.W, oquant.channel_absmax_cols(wl.calib), wl.alpha, 8, fmt, refine_iters=4)
    np.testing.assert_allclose(hp.errors, orc["errors"], rtol=1e-4)
    assert int(np.argmin(hp.errors)) == orc["best_iter"]
    assert _lib_split_error(hp, wl.W, fmt) == pytest.approx(hp.errors.min(), rel=1e-9)
    assert hp.errors.min() < hp.errors[0]
    for bad in (-1, 65):
        with pytest.raises(svdq.SvdqError):
            _refined_raw(wl.W, a, wl.alpha, 8, F, bad)


def _refined_raw(W, a, alpha, rank, F, iters):
    K, N = W.shape
    G = svdq.GROUP[F]
    s, inv = np.empty(K, np.float32), np.empty(K, np.float32)
    L1t, L2 = np.zeros((rank, K), np.uint16), np.zeros((rank, N), np.uint16)
    qW = np.empty((N, K // 2), np.uint8)
    sW = svdq._scale_buffer(K, N, F)[0]
    W = np.ascontiguousarray(W, dtype=np.uint16)
    svdq._check(svdq.lib().svdq_pack_weights_refined(K, N, svdq._ptr(W), svdq._ptr(a), float(alpha), rank, F, iters,
                                                     svdq._ptr(s), svdq._ptr(inv), svdq._ptr(L1t), svdq._ptr(L2),
                                                     svdq._ptr(qW), svdq._ptr(sW), None, None))


def test_concat_lora_bit_exact():
    wl = random_layer(16, 256, 72, 8, 91, lora_rank=4)
    orc = opack.pack_weights(wl.W, oquant.channel_absmax_cols(wl.X), wl.alpha, wl.rank, "int4")
    hp = svdq.HostPack(256, 72, 8, 0, orc["s32"], orc["inv_s32"], orc["L1_bits"].T.copy(), orc["L2_bits"],
                       orc["qW"], orc["sW"])
    for scale in (1.0, 0.75):
        f = svdq.concat_lora(hp, wl.lora_A, wl.lora_B, scale)
        o = opack.fold_lora(orc, wl.lora_A, wl.lora_B, scale)
        np.testing.assert_array_equal(f.L1t, o["L1_bits"].T)
        np.testing.assert_array_equal(f.L2, o["L2_bits"])


def test_prepare_lowrank_layouts():
    rng = np.random.default_rng(2)
    from bit_diffusion_model_amd.workloads import bf16_bits_from_f64
    L2 = bf16_bits_from_f64(rng.standard_normal((5, 40)))
    f = svdq.prepare_lowrank(L2)
    # fragment order: [column block of 32][k step of 16][lane = n % 32 + 32 (j / 8 % 2)][j % 8]
    assert f.shape == (64 * 16,)
    back = f.reshape(2, 1, 2, 32, 8).transpose(0, 3, 1, 2, 4).reshape(64, 16)  # [n][j]
    np.testing.assert_array_equal(back[:40, :5], L2.T)
    assert not back[:, 5:].any() and not back[40:].any()
    L2b = bf16_bits_from_f64(rng.standard_normal((37, 70)))  # three k steps, three column blocks
    f = svdq.prepare_lowrank(L2b)
    back = f.reshape(3, 3, 2, 32, 8).transpose(0, 3, 1, 2, 4).reshape(96, 48)
    np.testing.assert_array_equal(back[:70, :37], L2b.T)
    assert not back[:, 37:].any() and not back[70:].any()


def test_prepare_lowrank_down_layout():
    """L1f: for chunk c, rank tile t and lane l, the 16 channels 64 c + 16 (l >> 4) ..
    of rank row 16 t + (l & 15) at element ((c NT + t) 64 + l) 16; rows past the rank
    zero.  Checked by undoing the permutation with an independent index walk."""
    rng = np.random.default_rng(3)
    for rank, K in ((5, 128), (16, 192), (33, 256)):
        L1t = rng.integers(1, 1 << 16, size=(rank, K), dtype=np.uint16)
        f = svdq.prepare_lowrank_down(L1t)
        R16 = (rank + 15) // 16 * 16
        assert f.shape == (R16 * K,)
        full = f.reshape(K // 64, R16 // 16, 4, 16, 16)  # c, t, l >> 4, l & 15, e
        back = full.transpose(1, 3, 0, 2, 4).reshape(R16, K)  # [t, l & 15] rows, [c, l >> 4, e] columns
        np.testing.assert_array_equal(back[:rank], L1t)
        assert not back[rank:].any()
    with pytest.raises(svdq.SvdqError):
        svdq.prepare_lowrank_down(np.zeros((4, 96), np.uint16))  # K not a multiple of 64


def fp6_fields(words6):
    """[..., 6] uint32 words -> [..., 32] 6-bit fields, field f at bit 6 f of the 192-bit
    little-endian concatenation."""
    w = words6.astype(np.uint64)
    out = np.empty(words6.shape[:-1] + (32,), np.int64)
    for f in range(32):
        b, o = divmod(6 * f, 32)
        v = w[..., b] >> np.uint64(o)
        if o > 26:
            v = v | (w[..., b + 1] << np.uint64(32 - o))
        out[..., f] = (v & np.uint64(63)).astype(np.int64)
    return out


def fp6_codes(fields):
    """E2M3 fields with a zero exponent (sign bit 5, |q| in bits 0-2) -> codes q, in k
    order: field f of a half carries k = 16 (f & 1) + (f >> 1)."""
    assert not (fields & 0b011000).any(), "nonzero exponent bits"
    v = (fields & 7) * np.where(fields & 32, -1, 1)
    k = np.array([16 * (f & 1) + (f >> 1) for f in range(32)])
    out = np.empty_like(v)
    out[..., k] = v
    return out


Z0 = sum(3 << b for b in (3, 9, 15, 21, 27))
Z1 = sum(3 << b for b in (1, 7, 13, 19, 25)) | (1 << 31)


def test_prepare_weights_kernel_layout():
    """The kernel layout decodes back to the oracle's codes and scales: per 32-code group
    half four words w0..w3 give the six FP6 operand words f0 = w0 & ~Z0, f1 = w1 & ~Z1,
    f2 = (w0 & Z0) | (w1 & Z1) (f3..f5 likewise from w2, w3), whose fields are the codes
    as E2M3 values q / 8; the scales are the fp16 bits [K/64][Np], padded rows 0."""
    rng = np.random.default_rng(11)
    K, N = 256, 39  # N not a multiple of 4: padded scale rows
    R = (rng.standard_normal((K, N)) * 10.0 ** rng.uniform(-9, 2, (1, N))).astype(np.float32)
    R[:, 5] = 0.0
    R[64:128, 6] = 0.0
    codes, sc = opack.quantize_residual(R, "int4")
    qW = opack.pack_codes(codes, "int4")
    assert (sc.view(np.uint16) & 0x7C00 == 0).any(), "want subnormal fp16 scales in the case"
    qk, sk = svdq.prepare_weights(K, N, svdq.INT4_G64, qW, sc)
    # column pairs: byte b of column n at (n // 2) K + (b // 64) 128 + (n % 2) 64 + b % 64
    N2 = N + (N & 1)
    assert qk.size == N2 * K // 2
    pr = qk.reshape(N2 // 2, K // 128, 2, 64).transpose(0, 2, 1, 3).reshape(N2, K // 2)
    assert not pr[N:].any(), "phantom column must be zero"
    w = np.ascontiguousarray(pr[:N]).view("<u4").reshape(N, K // 32, 4)
    f = np.stack([w[..., 0] & ~np.uint32(Z0), w[..., 1] & ~np.uint32(Z1), (w[..., 0] & Z0) | (w[..., 1] & Z1),
                  w[..., 2] & ~np.uint32(Z0), w[..., 3] & ~np.uint32(Z1), (w[..., 2] & Z0) | (w[..., 3] & Z1)], -1)
    np.testing.assert_array_equal(fp6_codes(fp6_fields(f)).reshape(N, K), codes)
    Np = (N + 3) // 4 * 4
    G = K // 64
    assert sk.size == G * Np * 2
    sv = sk.view(np.uint16).reshape(G, Np)
    np.testing.assert_array_equal(sv[:, :N], sc.view(np.uint16))
    assert not sv[:, N:].any()
    c4, s4 = opack.quantize_residual(R, "mxfp4")
    qf, sf = svdq.prepare_weights(K, N, svdq.MXFP4_G32, opack.pack_codes(c4, "mxfp4"), s4)
    pf = qf.reshape(N2 // 2, K // 128, 2, 64).transpose(0, 2, 1, 3).reshape(N2, K // 2)
    np.testing.assert_array_equal(pf[:N], opack.pack_codes(c4, "mxfp4"))
    assert not pf[N:].any()
    sf = sf.reshape(K // 32, Np)
    np.testing.assert_array_equal(sf[:, :N], s4)
    assert np.all(sf[:, N:] == 127)


# ------------------------------------------------------------------ error paths

def _err():
    return svdq.lib().svdq_last_error().decode()


def test_pack_argument_errors():
    L = svdq.lib()
    W = np.zeros((256, 16), np.uint16)
    outs = [np.zeros(256, np.float32), np.zeros(256, np.float32), np.zeros((8, 256), np.uint16),
            np.zeros((8, 16), np.uint16), np.zeros((16, 128), np.uint8), np.zeros((4, 16), np.uint16)]
    P = [o.ctypes.data_as(ctypes.c_void_p) for o in outs]
    Wp = W.ctypes.data_as(ctypes.c_void_p)
    assert L.svdq_pack_weights(200, 16, Wp, None, 0.5, 8, 0, *P, None) == 1 and "multiple of 128" in _err()
    assert L.svdq_pack_weights(256, 16, Wp, None, 1.5, 8, 0, *P, None) == 1 and "alpha" in _err()
    assert L.svdq_pack_weights(256, 16, Wp, None, 0.5, 17, 0, *P, None) == 1 and "rank" in _err()
    assert L.svdq_pack_weights(256, 16, Wp, None, 0.5, 8, 7, *P, None) == 2
    assert L.svdq_pack_weights(256, 16, None, None, 0.5, 8, 0, *P, None) == 1
    W[3, 3] = 0x7FC0  # NaN
    assert L.svdq_pack_weights(256, 16, Wp, None, 0.5, 8, 0, *P, None) == 3 and "non-finite" in _err()
    assert L.svdq_concat_lora(256, 16, P[0], 100, P[2], P[3], 40, Wp, Wp, 1.0, P[2], P[3]) == 2


def test_device_entry_points_validate_on_host():
    L = svdq.lib()
    lay = svdq._Layer(256, 64, 8, 0, 16, 16, 16, 16, 16)  # fake aligned non-NULL pointers
    ref = ctypes.byref(lay)
    # M == 0 is a no-op that never touches the device
    assert L.svdq_quantize_act_lora_down(ref, 0, None, 256, 0, None, None, None, None) == 0
    assert L.svdq_gemm_w4a4_lora_up(ref, 0, 0, None, None, None, None, 64, 0, None, 0, None) == 0
    assert L.svdq_quantize_act_lora_down(None, 4, None, 256, 0, None, None, None, None) == 1
    bad = svdq._Layer(200, 64, 8, 0, 16, 16, 16, 16, 16)
    assert L.svdq_quantize_act_lora_down(ctypes.byref(bad), 4, 16, 256, 0, 16, 16, 16, None) == 1
    big = svdq._Layer(256, 64, 129, 0, 16, 16, 16, 16, 16)
    assert L.svdq_gemm_w4a4_lora_up(ctypes.byref(big), 4, 0, 16, 16, 16, 16, 64, 0, None, 0, None) == 2
    assert L.svdq_quantize_act_lora_down(ref, 4, 16, 100, 0, 16, 16, 16, None) == 1 and "ldx" in _err()
    assert L.svdq_quantize_act_lora_down(ref, 4, 18, 256, 0, 16, 16, 16, None) == 1 and "aligned" in _err()
    assert L.svdq_quantize_act_lora_down(ref, 4, 16, 256, 2, 16, 16, 16, None) == 2 and "form" in _err()
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 0, 16, 16, 16, 16, 32, 0, None, 0, None) == 1 and "ldy" in _err()
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 0, 16, 16, 16, 16, 1 << 23, 0, None, 0, None) == 2 and "ldy" in _err()
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 0, 16, 16, 16, 16, 64, 5, None, 0, None) == 2
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 7, 16, 16, 16, 16, 64, 0, None, 0, None) == 2 and "form" in _err()
    unal = svdq._Layer(256, 64, 8, 0, 16, 16, 16, 16, 18)
    assert L.svdq_gemm_w4a4_lora_up(ctypes.byref(unal), 4, 0, 16, 16, 16, 16, 64, 0, None, 0, None) == 1 and "sW" in _err()
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 0, 16, 16, 16, 16, 64, 0, 8, 1 << 20, None) == 1 and "workspace" in _err()
    assert L.svdq_linear_forward(ref, 4, 16, 256, 16, 64, 0, 256, 10, None) == 1 and "workspace" in _err()
    assert L.svdq_linear_forward_unfused(ref, 4, 16, 256, 16, 64, 0, 256, 10, None) == 1 and "workspace" in _err()
    assert L.svdq_linear_forward_unfused(ref, 0, 16, 256, 16, 64, 0, None, 0, None) == 0  # M = 0: no-op
    assert L.svdq_linear_forward_unfused(ref, -1, 16, 256, 16, 64, 0, None, 0, None) == 1
    assert L.svdq_debug_group_sums(ref, 4, 1, 16, 0, 0, 5, 4, 16, None) == 1 and "window" in _err()
    assert L.svdq_debug_group_sums(ref, 4, 0, 16, 0, 0, 5, 4, 16, None) == 1 and "window" in _err()
    assert L.svdq_debug_group_sums(ref, 4, 3, 16, 0, 0, 4, 4, 16, None) == 2 and "form" in _err()
    # the output rows of a tile are addressed through a 32-bit range: ldy below 2^22
    assert L.svdq_gemm_w4a4_lora_up(ref, 4, 1, 16, 16, 16, 16, 1 << 22, 0, None, 0, None) == 2 and "ldy" in _err()
    # MMA form: FP6 operand words (M*K bytes), fp16 scales (2 bytes per group and row),
    # 2*R16 bf16 per row, rows rounded up to 32
    assert L.svdq_workspace_bytes(ref, 100) >= 100 * 256 + 4 * 100 * 2 + 128 * 16 * 4
    # kernel 1 in one pass at short K; the query refuses what the workspace size refuses
    assert L.svdq_forward_k1_parts(ref, 100) == 1
    assert L.svdq_forward_k1_parts(None, 100) == 0 and L.svdq_forward_k1_parts(ref, -1) == 0
    bad = svdq._Layer(100, 64, 8, 0, 16, 16, 16, 16, 16)  # K not a multiple of 128
    assert L.svdq_forward_k1_parts(ctypes.byref(bad), 4) == 0


def test_mlp_entry_points_validate_on_host():
    L = svdq.lib()
    fc1 = svdq._Layer(256, 384, 8, 0, 16, 16, 16, 16, 16)  # fake aligned non-NULL pointers
    fc2 = svdq._Layer(384, 64, 8, 0, 16, 16, 16, 16, 16)
    r1, r2 = ctypes.byref(fc1), ctypes.byref(fc2)
    # fc1.N must equal fc2.K
    assert L.svdq_mlp_forward(r1, r1, 4, 16, 256, 16, 64, 0, 0, 256, 1 << 30, None) == 1 and "fc2's K" in _err()
    assert L.svdq_mlp_forward(r1, r2, 4, 16, 256, 16, 64, 0, 5, 256, 1 << 30, None) == 2 and "mode" in _err()
    assert L.svdq_mlp_forward(r1, r2, 0, 16, 256, 16, 64, 0, 0, None, 0, None) == 0  # M = 0: no-op
    assert L.svdq_mlp_forward(r1, r2, 4, 16, 256, 16, 64, 0, 0, 256, 10, None) == 1 and "workspace" in _err()
    # the chained pair runs INT4 layers; the separate mode takes any format
    fx = svdq._Layer(384, 64, 8, 1, 16, 16, 16, 16, 16)
    assert L.svdq_mlp_forward(r1, ctypes.byref(fx), 4, 16, 256, 16, 64, 0, 0, 256, 1 << 30, None) == 2
    assert L.svdq_mlp_chain_gemm(r1, ctypes.byref(fx), 4, 16, 16, 16, 16, 16, 16, None, 0, None) == 2
    assert L.svdq_mlp_chain_gemm(r1, r2, 4, 16, 16, 16, 16, 16, None, None, 0, None) == 1 and "lora_part" in _err()
    assert L.svdq_mlp_chain_gemm(r1, r2, 4, 16, 16, 16, 16, 16, 16, 16, 100, None) == 1 and "ldh" in _err()
    assert L.svdq_mlp_chain_reduce(r1, r2, 4, None, 16, None) == 1
    # workspace sizes: chained holds fc2's activation side, fc1's and the partials
    # (384/128 tiles x M x 16 fp32); separate holds the bf16 hidden M x 384
    M = 100
    wc = L.svdq_mlp_workspace_bytes(r1, r2, M, 0)
    ws = L.svdq_mlp_workspace_bytes(r1, r2, M, 1)
    assert wc >= L.svdq_workspace_bytes(r2, M) + M * 256 + 3 * M * 16 * 4
    assert ws >= M * 384 * 2 + max(L.svdq_workspace_bytes(r1, M), L.svdq_workspace_bytes(r2, M))
    assert L.svdq_mlp_workspace_bytes(r1, r2, M, 3) == 0
    # the unfused forward has no GELU output
    assert L.svdq_linear_forward_unfused(r1, 4, 16, 256, 16, 384, 2, 256, 1 << 30, None) == 2 and "GELU" in _err()


def test_w4a16_gemm_validates_on_host():
    """The weight-only baseline's argument checks (fake aligned device pointers: every call
    below is refused before any launch)."""
    L = svdq.lib()
    g = L.svdq_w4a16_gemm
    # M, K, N, X, ldx, qW, sW, Y, ldy, ydtype, stream
    assert g(0, 256, 64, 16, 256, 16, 16, 16, 64, 0, None) == 0  # M = 0: no-op
    assert g(-1, 256, 64, 16, 256, 16, 16, 16, 64, 0, None) == 1
    assert g(4, 100, 64, 16, 256, 16, 16, 16, 64, 0, None) == 1 and "multiple of 64" in _err()
    assert g(4, 256, 0, 16, 256, 16, 16, 16, 64, 0, None) == 1
    assert g(4, 256, 64, None, 256, 16, 16, 16, 64, 0, None) == 1 and "non-NULL" in _err()
    assert g(4, 256, 64, 16, 128, 16, 16, 16, 64, 0, None) == 1 and "ldx" in _err()
    assert g(4, 256, 64, 16, 260, 16, 16, 16, 64, 0, None) == 1 and "ldx" in _err()
    assert g(4, 256, 64, 16, 256, 16, 16, 16, 32, 0, None) == 1 and "ldy" in _err()
    assert g(4, 256, 64, 16, 256, 16, 16, 16, 64, 2, None) == 2 and "dtype" in _err()
    assert g(4, 256, 64, 16, 1 << 22, 16, 16, 16, 64, 0, None) == 2 and "2^22" in _err()
    assert g(4, 256, 64, 18, 256, 16, 16, 16, 64, 0, None) == 1 and "aligned" in _err()
    assert g(4, 256, 64, 16, 256, 24, 16, 16, 64, 0, None) == 1 and "aligned" in _err()
    assert g(4, 256, 64, 16, 256, 16, 16, 18, 64, 0, None) == 1 and "aligned" in _err()  # fp32 Y


@pytest.mark.parametrize("fmt", [svdq.INT4_G64, svdq.NVFP4_G16])
def test_pack_save_load_round_trip(fmt, tmp_path):
    """The offline artifacts written to one .npz and read back are the same bits."""
    wl = random_layer(48, 256, 96, 8, 31)
    p = svdq.pack_weights(wl.W, svdq.act_absmax(wl.X), wl.alpha, wl.rank, fmt, want_R=True)
    path = str(tmp_path / "pack.npz")
    svdq.save_pack(p, path)
    q = svdq.load_pack(path)
    assert (q.K, q.N, q.rank, q.fmt) == (p.K, p.N, p.rank, p.fmt)
    assert (q.tscale_w, q.tscale_x) == (p.tscale_w, p.tscale_x)
    for k in ("s", "inv_s", "L1t", "L2", "qW", "sW", "R"):
        a, b = getattr(p, k), getattr(q, k)
        assert a.dtype == b.dtype and a.shape == b.shape and a.tobytes() == b.tobytes(), k
    assert q.errors is None


def test_launch_failure_reports_hip_error():
    """A launch that the HIP runtime refuses (here: no device in this container) returns
    SVDQ_EHIP with the runtime's message, and nothing aborts."""
    import torch

    if torch.cuda.is_available():
        pytest.skip("needs a host without a visible GPU")
    L = svdq.lib()
    lay = svdq._Layer(256, 64, 8, 0, 16, 16, 16, 16, 16)
    assert L.svdq_quantize_act_lora_down(ctypes.byref(lay), 4, 16, 256, 1, 16, 16, 16, None) == 4
    assert "kernel 1 launch" in _err()
    assert L.svdq_w4a16_gemm(4, 256, 64, 16, 256, 16, 16, 16, 64, 0, None) == 4
    assert "weight-only kernel launch" in _err()
