"""GPU parity of the HIP path against the oracle on small and ragged shapes.

Bar: bit-exact 4-bit codes, scales and INT4 integer group sums; lora_act within the
arithmetic's error budget; Y within 2e-2 x RMS of the oracle output (fp32 output).
Shapes span several output tiles and 16-token kernel-1 tiles with ragged tails, K from
128 (the minimum) upward, ranks 0 / 1 / 8 / 48 / 128, and K long enough for kernel 2 to
split its last round along K.

Every output, activation and workspace buffer is filled with 0xFF bytes (NaN) before
the kernels run, so an element no kernel wrote cannot pass as a value left over from
an earlier allocation.  The exact integer group sums are taken from the forward's own
kernel 2 twice: through its debug instance (same schedule, loads, LDS layout and
group-sum MFMA; each group's result stored) and through the timed instance itself, fed
weight scales 1.0 and activation scales 1.0 on one group and 0.0 on the others, so that
its output is exactly that group's integer sums (and with 1.0 everywhere their sum).
"""
import numpy as np
import pytest

from gpu_helpers import (TOL_Y, assert_finite, bf16_rne_bits, decode_lora_mma, decode_mma, forward_sentinel,
                         layer_from_oracle, log, lora_bound, mma_scales_int4, oracle_k1, oracle_pack, rel_err,
                         sentinel_act, sentinel_gemm_ws, sentinel_out, to_dev_bf16, unit_scale_layer)

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import make, random_layer
from oracle import forward as oforward

pytestmark = pytest.mark.gpu

SHAPES = [  # M, K, N, rank, fmt
    (64, 256, 256, 8, "int4"),
    (1, 128, 1, 0, "int4"),
    (17, 128, 33, 1, "int4"),
    (300, 384, 520, 8, "int4"),
    (530, 256, 257, 48, "int4"),
    (33, 128, 160, 128, "int4"),
    (64, 256, 256, 8, "mxfp4"),
    (17, 128, 33, 1, "mxfp4"),
    (300, 384, 520, 16, "mxfp4"),
    # K long enough that kernel 2 splits its tiles along K (few tiles, >= 8 K steps)
    (200, 1024, 300, 8, "int4"),
    (130, 768, 260, 16, "mxfp4"),
    # the group-16 two-level-scale variant
    (64, 256, 256, 8, "nvfp4"),
    (17, 128, 33, 1, "nvfp4"),
    (300, 384, 520, 16, "nvfp4"),
    (200, 1024, 300, 48, "nvfp4"),
]


def _ids(s):
    return "M{}_K{}_N{}_r{}_{}".format(*s)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_kernel1_codes_scales_lora(shape):
    M, K, N, r, fmt = shape
    log(f"k1 {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    qX, sX, la = lay.quantize_act(X, out=sentinel_act(lay, M, svdq.ACT_PACKED))
    import torch

    torch.cuda.synchronize()
    Xh, codes, sc, qX_ref, sX_ref, la_ref = oracle_k1(wl.X, p)
    np.testing.assert_array_equal(qX.cpu().numpy(), qX_ref)
    np.testing.assert_array_equal(sX.cpu().numpy().view(sX_ref.dtype), sX_ref)
    if r:
        la_g = la.cpu().numpy().astype(np.float64)
        assert la_g.shape[1] == svdq.r16(r) and not la_g[:, r:].any()
        assert np.all(np.abs(la_g[:, :r] - la_ref) <= lora_bound(Xh, p["L1b"]))
    # the MMA form: the same codes and scales re-encoded, lora_act as the bf16 hi/lo
    # split of the very fp32 values above
    qm, sm, lam = lay.quantize_act(X, out=sentinel_act(lay, M, svdq.ACT_MMA), form=svdq.ACT_MMA)
    c_m, s_m, hi, lo = decode_mma(qm, sm, lam, fmt, K, r, M=M)
    if fmt == "int4":
        np.testing.assert_array_equal(c_m, codes)
        np.testing.assert_array_equal(s_m, sX_ref.view(np.float16).astype(np.float64))
    else:
        np.testing.assert_array_equal(c_m, qX_ref)
        np.testing.assert_array_equal(s_m, sX_ref)
    if r:
        v = la.cpu().numpy()
        np.testing.assert_array_equal(hi, bf16_rne_bits(v))
        rem = v - (hi.astype(np.uint32) << 16).view(np.float32)
        np.testing.assert_array_equal(lo, bf16_rne_bits(rem))


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[4] == "int4"], ids=_ids)
@pytest.mark.parametrize("form", [svdq.ACT_MMA, svdq.ACT_PACKED], ids=["mma", "packed"])
def test_kernel2_group_sums_exact(shape, form):
    """Exact integer group sums from kernel 2's debug instance: form MMA is the forward's
    streamed kernel (same schedule and K split), form PACKED the packed-form kernel."""
    import torch

    M, K, N, r, fmt = shape
    log(f"groupsums {_ids(shape)} form {form}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    qX, sX, la = lay.quantize_act(to_dev_bf16(wl.X), out=sentinel_act(lay, M, form), form=form)
    _, codes, _, _, _, _ = oracle_k1(wl.X, p)
    I_ref = oforward.group_sums(codes, p["codesW"], 64)
    out = torch.full((K // 64, M, N), -(2 ** 31), dtype=torch.int32, device="cuda:0")
    I = lay.group_sums(qX, 0, 0, M, N, form=form, out=out).cpu().numpy()
    np.testing.assert_array_equal(I, I_ref)
    if M > 2 and N > 3:  # an interior window
        I2 = lay.group_sums(qX, M // 3, N // 4, M - M // 3, N - N // 4, form=form).cpu().numpy()
        np.testing.assert_array_equal(I2, I_ref[:, M // 3:, N // 4:])


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[4] == "int4"], ids=_ids)
def test_forward_kernel2_exact_with_unit_scales(shape):
    """The forward's kernel 2 instance itself (the one svdq_linear_forward times), on kernel
    1's MMA-form codes, with weight scales 1.0: activation scales 1.0 on group g only give
    Y = I_g exactly (every group, so a K-split tail is covered), and 1.0 everywhere give
    Y = sum_g I_g = the plain integer product of the codes."""
    import torch

    M, K, N, r, fmt = shape
    log(f"unit scales {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = unit_scale_layer(p)
    qX, _, _ = lay.quantize_act(to_dev_bf16(wl.X), out=sentinel_act(lay, M, svdq.ACT_MMA), form=svdq.ACT_MMA)
    _, codes, _, _, _, _ = oracle_k1(wl.X, p)
    I_ref = oforward.group_sums(codes, p["codesW"], 64)
    G = K // 64
    gws = sentinel_gemm_ws(lay, M, svdq.ACT_MMA)
    for g in range(G):
        Y = lay.gemm(qX, mma_scales_int4(M, K, [g]), None, out=sentinel_out(M, N), form=svdq.ACT_MMA,
                     workspace=gws).cpu().numpy()
        np.testing.assert_array_equal(Y, I_ref[g].astype(np.float32))
    Y = lay.gemm(qX, mma_scales_int4(M, K, range(G)), None, out=sentinel_out(M, N), form=svdq.ACT_MMA,
                 workspace=gws).cpu().numpy()
    np.testing.assert_array_equal(Y, oforward.code_product(codes, p["codesW"]).astype(np.float32))
    if K >= 768:
        assert gws is not None, "expected kernel 2 to split this shape"


@pytest.mark.parametrize("shape", [(100, 8320, 96, 32, "int4"), (100, 8192, 96, 32, "mxfp4"),
                                   (37, 8192, 64, 16, "nvfp4"), (50, 8192, 64, 0, "int4")], ids=_ids)
def test_forward_long_k_split(shape):
    """At K >= 8192 (and at most two 16-token blocks per CU) the forward cuts kernel 1's
    chunks along K into 4 ranges (K = 8320: 130 chunks, ranges of 32 and 33) and adds the
    ranges' down-projection sums in a second step.  Codes and scales stay bit-exact;
    lora_act keeps the arithmetic's error budget (only the order of its fp32 additions
    differs from the single-pass kernel 1); Y meets the bar; repeated calls give the same
    bits.  At rank 0 the standalone kernel 1 takes the same cut, so the separate calls
    match the forward bit for bit."""
    M, K, N, r, fmt = shape
    log(f"forward, kernel 1 cut along K: {_ids(shape)}")
    _check_k1_cut_forward(M, K, N, r, fmt, 4)


@pytest.mark.parametrize("shape", [(0, 256, 96, 0, "int4"), (-3, 384, 64, 0, "int4"), (5, 256, 64, 0, "mxfp4"),
                                   (-1, 256, 64, 0, "nvfp4"), (2, 256, 64, 32, "int4")],
                         ids=lambda s: f"tail{s[0]:+d}_K{s[1]}_N{s[2]}_r{s[3]}_{s[4]}")
def test_forward_tail_cut(shape):
    """At short K and rank 0, when the 16-token blocks leave a last round of one block per
    CU at most half full (here 16 (CUs + CUs / 8) tokens plus the offset: a ragged last
    block or a round of CUs / 8 + 1 blocks), every kernel-1 launch keeps the full rounds'
    blocks whole and cuts only the last round's blocks along K, into min(8, CUs / blocks,
    K / 64) ranges (K = 384: 6 ranges of one chunk).  Codes and scales bit-exact, Y at the
    bar, bitwise repeatable and bit-identical to the separate calls.  At rank > 0 the
    forward stays one pass (the second step would cost what the balance gains)."""
    import torch

    off, K, N, r, fmt = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    M = 16 * (cus + cus // 8) + off
    rem = (M + 15) // 16 - cus
    parts = min(8, cus // rem, K // 64) if r == 0 else 1
    log(f"forward, kernel 1 cut in its last round: M={M} ({rem} blocks past {cus} CUs, {parts} ranges) K={K} "
        f"N={N} r={r} {fmt}")
    _check_k1_cut_forward(M, K, N, r, fmt, parts)


def _check_k1_cut_forward(M, K, N, r, fmt, parts):
    import torch

    wl = random_layer(M, K, N, r, 9100 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    assert lay.forward_k1_parts(M) == parts
    assert lay.forward_k1_parts(64 * torch.cuda.get_device_properties(0).multi_processor_count) == 1
    X = to_dev_bf16(wl.X)
    Yd, ws = forward_sentinel(lay, X)
    assert_finite(Yd)
    Yref = oforward.forward(wl.X, p)["Y"]
    e = rel_err(Yd.cpu().numpy().astype(np.float64), Yref)
    log(f"  max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    Xh, _, _, qX_ref, sX_ref, la_ref = oracle_k1(wl.X, p)
    Mp = (M + 3) // 4 * 4
    if fmt == "int4":
        sx0 = (M * K + 255) // 256 * 256
        la0 = sx0 + ((K // 64) * Mp * 2 + 255) // 256 * 256
        c_m, s_m, hi, lo = decode_mma(ws[:M * K].view(M, K), ws[sx0:sx0 + (K // 64) * Mp * 2], ws[la0:], fmt, K, r,
                                      M=M)
        _, codes_ref, _, _, _, _ = oracle_k1(wl.X, p)
        np.testing.assert_array_equal(c_m, codes_ref)
        np.testing.assert_array_equal(s_m, sX_ref.view(np.float16).astype(np.float64))
    else:
        G = 32 if fmt == "mxfp4" else 16
        nq = (M + 1) // 2 * 2 * (K // 2)
        sx0 = (nq + 255) // 256 * 256
        la0 = sx0 + ((K // G) * Mp + 255) // 256 * 256
        c_m, s_m, hi, lo = decode_mma(ws[:M * (K // 2)].view(M, K // 2), ws[sx0:sx0 + (K // G) * Mp], ws[la0:], fmt,
                                      K, r, M=M)
        np.testing.assert_array_equal(c_m, qX_ref)
        np.testing.assert_array_equal(s_m, sX_ref)
    if r > 0:
        # hi + lo carries the fp32 sum to 2^-17 of its size
        v = (hi.astype(np.uint32) << 16).view(np.float32).astype(np.float64) + \
            (lo.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        R16 = (r + 15) // 16 * 16
        assert not v[:, r:].any()
        err = np.abs(v[:, :r] - la_ref)
        assert np.all(err <= lora_bound(Xh, p["L1b"]) + 2.0 ** -16 * np.abs(la_ref)), float(err.max())
        assert v.shape == (M, R16)
    # against the two kernels called one after the other (kernel 1 in one pass)
    qX, sX, la = lay.quantize_act(X, out=sentinel_act(lay, M, svdq.ACT_MMA), form=svdq.ACT_MMA)
    Y2 = lay.gemm(qX, sX, la, out=sentinel_out(M, N), form=svdq.ACT_MMA,
                  workspace=sentinel_gemm_ws(lay, M, svdq.ACT_MMA)).cpu().numpy().astype(np.float64)
    Yg = Yd.cpu().numpy().astype(np.float64)
    e2 = rel_err(Yg, Y2)
    log(f"  forward against the separate calls: max|dY|/RMS = {e2:.2e}")
    if r == 0:  # no sums to add across the ranges: the standalone call takes the same cut
        np.testing.assert_array_equal(Yg, Y2)
    # the same fp32 terms of the down projection added in another order (the outlier
    # channels make single terms large against the sums: measured 2.5e-5 at K = 8320)
    assert e2 <= 1e-4
    Y3 = lay.forward(X, workspace=ws)
    assert torch.equal(Y3, Yd)


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_forward_matches_oracle(shape):
    M, K, N, r, fmt = shape
    log(f"forward {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    Yd, ws = forward_sentinel(lay, to_dev_bf16(wl.X))
    assert_finite(Yd)
    Y = Yd.cpu().numpy().astype(np.float64)
    Yref = oforward.forward(wl.X, p)["Y"]
    e = rel_err(Y, Yref)
    log(f"  max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    # the forward keeps the activation side in MMA form at the start of its workspace:
    # codes and scales bit-exact
    Mp = (M + 3) // 4 * 4
    _, codes_ref, _, qX_ref, sX_ref, _ = oracle_k1(wl.X, p)
    if fmt == "int4":
        sx0 = (M * K + 255) // 256 * 256
        codes, sv = decode_mma(ws[:M * K].view(M, K), ws[sx0:sx0 + (K // 64) * Mp * 2], None, "int4", K, 0, M=M)[:2]
        np.testing.assert_array_equal(codes, codes_ref)
        np.testing.assert_array_equal(sv, sX_ref.view(np.float16).astype(np.float64))
    else:
        nq = (M + 1) // 2 * 2 * (K // 2)
        sx0 = (nq + 255) // 256 * 256
        G = 32 if fmt == "mxfp4" else 16
        rows, sb = decode_mma(ws[:M * (K // 2)].view(M, K // 2), ws[sx0:sx0 + (K // G) * Mp], None, fmt, K, 0,
                              M=M)[:2]
        np.testing.assert_array_equal(rows, qX_ref)
        np.testing.assert_array_equal(sb, sX_ref)
    # the two kernels called separately in MMA form, kernel 2 with its split workspace,
    # give the same bits as the forward; without the workspace (no split) the same bar
    X = to_dev_bf16(wl.X)
    qX, sX, la = lay.quantize_act(X, out=sentinel_act(lay, M, svdq.ACT_MMA), form=svdq.ACT_MMA)
    gws = sentinel_gemm_ws(lay, M, svdq.ACT_MMA)
    Y2 = lay.gemm(qX, sX, la, out=sentinel_out(M, N), form=svdq.ACT_MMA, workspace=gws).cpu().numpy()
    np.testing.assert_array_equal(Y2, Y.astype(np.float32))
    Ynd = lay.gemm(qX, sX, la, out=sentinel_out(M, N), form=svdq.ACT_MMA)
    assert_finite(Ynd)
    en = rel_err(Ynd.cpu().numpy().astype(np.float64), Yref)
    log(f"  unsplit kernel 2 max|err|/RMS = {en:.3e} (split workspace {0 if gws is None else gws.numel()} B)")
    assert en <= TOL_Y
    if K >= 768:
        assert gws is not None, "expected kernel 2 to split this shape"
    # the packed form meets the same bar (kernel 2 on the NVFP4 format takes the MMA form only)
    if fmt == "nvfp4":
        with pytest.raises(svdq.SvdqError):
            lay.gemm(qX, sX, la, out=sentinel_out(M, N), form=svdq.ACT_PACKED)
        return
    qX, sX, la = lay.quantize_act(X, out=sentinel_act(lay, M, svdq.ACT_PACKED))
    Ypd = lay.gemm(qX, sX, la, out=sentinel_out(M, N))
    assert_finite(Ypd)
    ep = rel_err(Ypd.cpu().numpy().astype(np.float64), Yref)
    log(f"  packed form max|err|/RMS = {ep:.3e}")
    assert ep <= TOL_Y


def _fwd(lay, X, ydtype=svdq.F32, fused=True):
    """The forward on sentinel-filled Y and workspace; every output written and finite."""
    Y, _ = forward_sentinel(lay, X, ydtype, fused)
    assert_finite(Y)
    return Y


def test_tiny_config_c0():
    wl = make("C0")
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    Y = _fwd(lay, X).cpu().numpy().astype(np.float64)
    Yref = oforward.forward(wl.X, p)["Y"]
    e = rel_err(Y, Yref)
    log(f"C0 max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y


def test_rank0_and_zero_residual():
    wl = random_layer(200, 256, 300, 8, 99, x_out=3)
    p0 = oracle_pack(wl, rank=0)
    Y = _fwd(layer_from_oracle(p0), to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
    assert rel_err(Y, oforward.forward(wl.X, p0)["Y"]) <= TOL_Y
    p = dict(oracle_pack(wl))
    p["codesW"] = np.zeros_like(p["codesW"])
    p["qW"] = np.zeros_like(p["qW"])
    Y = _fwd(layer_from_oracle(p), to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
    ref = oforward.forward(wl.X, p)["Y"]
    assert rel_err(Y, ref) <= 1e-3  # only the low-rank branch remains: fp32-accurate


def test_bf16_output_and_determinism():
    wl = random_layer(257, 256, 300, 8, 5, x_out=3)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    Y32 = _fwd(lay, X)
    Yb = _fwd(lay, X, ydtype=svdq.BF16).float().cpu().numpy().astype(np.float64)
    ref = oforward.forward(wl.X, p)["Y"]
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(Yb - ref) <= 2.0 ** -8 * np.abs(ref) + TOL_Y * rms)
    for _ in range(5):
        assert np.array_equal(_fwd(lay, X).cpu().numpy(), Y32.cpu().numpy())


def test_strided_activation_rows():
    import torch

    wl = random_layer(40, 256, 96, 8, 12, x_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    Xp = np.zeros((40, 256 + 64), np.uint16)
    Xp[:, :256] = wl.X
    Xd = to_dev_bf16(Xp)[:, :256]
    assert Xd.stride(0) == 320
    Y = _fwd(lay, Xd).cpu().numpy().astype(np.float64)
    assert rel_err(Y, oforward.forward(wl.X, p)["Y"]) <= TOL_Y


def _ws_lora_region(M, K, rank, fmt):
    """Byte range of lora_act in the forward workspace: MMA-form qX, sX, lora_act in that
    order, each starting on a 256-byte boundary."""
    rup = lambda x: (x + 255) // 256 * 256
    Mp = (M + 3) // 4 * 4
    qx = M * K if fmt == "int4" else (M + 1) // 2 * 2 * (K // 2)
    # scale planes: INT4 fp16 [K/64][Mp], MXFP4 E8M0 [K/32][Mp], NVFP4 E4M3 [K/64][Mp][4]
    sx = {"int4": (K // 64) * Mp * 2, "mxfp4": (K // 32) * Mp, "nvfp4": (K // 16) * Mp}[fmt]
    off = rup(qx) + rup(sx)
    return off, off + (M + 31) // 32 * 32 * ((rank + 15) // 16 * 16) * 4


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_unfused_baseline_matches_oracle(shape):
    """svdq_linear_forward_unfused: the low-rank branch as kernels of its own meets the
    forward's bar, its lora_act is the fused kernel 1's bit for bit, and with rank 0 it is
    the fused forward."""
    M, K, N, r, fmt = shape
    log(f"unfused {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    Yref = oforward.forward(wl.X, p)["Y"]
    Yfd, wsf = forward_sentinel(lay, X)
    Yud, wsu = forward_sentinel(lay, X, fused=False)
    assert_finite(Yfd)
    assert_finite(Yud)
    Yf, Yu = Yfd.cpu().numpy(), Yud.cpu().numpy()
    e = rel_err(Yu.astype(np.float64), Yref)
    log(f"  max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    if r == 0:
        np.testing.assert_array_equal(Yu, Yf)
    else:
        a, b = _ws_lora_region(M, K, r, fmt)  # rows past M are not written: compare rows < M
        for u, f in zip(decode_lora_mma(wsu[a:b], M, r), decode_lora_mma(wsf[a:b], M, r)):
            np.testing.assert_array_equal(u, f)
        # the same two fp32 terms added in another order
        rms = np.sqrt(np.mean(Yref ** 2))
        assert np.abs(Yu.astype(np.float64) - Yf).max() <= 1e-5 * rms
    # bf16 output: the 4-bit term is rounded to bf16 in Y, then Y + lora_act L2 again
    # (each rounding within 2^-8 relative: half a bf16 ulp), on top of the forward's bar
    Yb = _fwd(lay, X, ydtype=svdq.BF16, fused=False).float().cpu().numpy().astype(np.float64)
    o = oforward.forward(wl.X, p)
    Yres = Yref - (o["lora_act"] @ np.asarray(p["L2b"], np.float64) if r else 0.0)
    rms = np.sqrt(np.mean(Yref ** 2))
    excess = np.abs(Yb - Yref) - (2.0 ** -8 * (np.abs(Yres) + np.abs(Yref)) + TOL_Y * rms)
    log(f"  bf16 max|err|/RMS = {rel_err(Yb, Yref):.3e}, worst excess over the bound {excess.max() / rms:.3e} RMS")
    assert excess.max() <= 0


def test_refined_pack_forward():
    """A pack from the refined split runs through the same kernels to the same bar."""
    from oracle import pack as opack, quant as oquant

    wl = random_layer(300, 384, 520, 16, 77, fmt="int4", x_out=3, w_out=2)
    p = opack.pack_weights(wl.W, oquant.channel_absmax_cols(wl.calib), wl.alpha, 16, "int4", refine_iters=3)
    log(f"refined pack: errors {p['errors']}, kept iterate {p['best_iter']}")
    lay = layer_from_oracle(p)
    Y = _fwd(lay, to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
    e = rel_err(Y, oforward.forward(wl.X, p)["Y"])
    log(f"  max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y


@pytest.mark.parametrize("ydtype", [svdq.F32, svdq.BF16], ids=["f32", "bf16"])
def test_unfused_strided_rows_and_padded_output(ydtype):
    """Both forwards with X rows strided past K and Y rows padded past N: the padding
    columns of Y are never written (kernel 2's store and the up-projection kernel's
    read-modify-write both mask columns >= N), and the two agree."""
    import torch

    M, K, N, r = 70, 256, 100, 16
    wl = random_layer(M, K, N, r, 21, x_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    Xp = np.zeros((M, K + 64), np.uint16)
    Xp[:, :K] = wl.X
    Xd = to_dev_bf16(Xp)[:, :K]
    dt = torch.float32 if ydtype == svdq.F32 else torch.bfloat16
    outs = []
    for fused in (True, False):
        Yfull = torch.full((M, N + 28), 7.0, dtype=dt, device="cuda:0")
        Yfull[:, :N] = float("nan")  # the sentinel: every element the forward must write
        Y = Yfull[:, :N]
        lay.forward(Xd, ydtype=ydtype, out=Y, fused=fused)
        assert bool((Yfull[:, N:] == 7.0).all()), "padding columns written"
        assert_finite(Y)
        outs.append(Y.float().cpu().numpy().astype(np.float64))
    Yref = oforward.forward(wl.X, p)["Y"]
    rms = np.sqrt(np.mean(Yref ** 2))
    for Yg in outs:
        if ydtype == svdq.F32:
            assert rel_err(Yg, Yref) <= TOL_Y
        else:  # bf16 output: half an ulp per rounding (two for the unfused form), on top of the bar
            assert np.all(np.abs(Yg - Yref) <= 2.0 ** -7 * np.abs(Yref) + TOL_Y * rms)
    if ydtype == svdq.F32:
        assert np.abs(outs[0] - outs[1]).max() <= 1e-5 * rms


def test_full_size_forward_bitwise_deterministic():
    """Ten forwards of the FLUX QKV layer in the bench's launch configuration (the K split
    of the last round included) give the same bits; so do ten of the MXFP4 layer."""
    import torch

    for name in ("C1", "C3"):
        wl = make(name)
        hp = svdq.pack_weights(wl.W, svdq.act_absmax(wl.calib), wl.alpha, wl.rank, svdq.FMT[wl.fmt])
        lay = svdq.PackedLinear.from_host_pack(hp)
        X = to_dev_bf16(wl.X)
        ws = lay.workspace(wl.M)
        Y0 = lay.forward(X, workspace=ws).clone()
        for _ in range(9):
            Y = lay.forward(X, workspace=ws)
            assert torch.equal(Y, Y0), name
        log(f"  {name}: 10 forwards bit-identical")
