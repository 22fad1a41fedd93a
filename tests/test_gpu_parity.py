"""GPU parity of the HIP path against the oracle on small and ragged shapes.

Bar: bit-exact 4-bit codes, scales and INT4 integer group sums; lora_act within the
arithmetic's error budget; Y within 2e-2 x RMS of the oracle output (fp32 output).
Shapes span several 256 x 256 output tiles and 16-token kernel-1 tiles with ragged
tails, K from 128 (the minimum) upward, ranks 0 / 1 / 8 / 48 / 128.
"""
import numpy as np
import pytest

from gpu_helpers import (TOL_Y, bf16_rne_bits, decode_lora_mma, decode_mma, layer_from_oracle, log, lora_bound,
                         oracle_k1, oracle_pack, rel_err, to_dev_bf16)

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
    qX, sX, la = lay.quantize_act(X)
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
    qm, sm, lam = lay.quantize_act(X, form=svdq.ACT_MMA)
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
def test_kernel2_group_sums_exact(shape):
    M, K, N, r, fmt = shape
    log(f"groupsums {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    qX, sX, la = lay.quantize_act(to_dev_bf16(wl.X))
    _, codes, _, _, _, _ = oracle_k1(wl.X, p)
    I_ref = oforward.group_sums(codes, p["codesW"], 64)
    I = lay.group_sums(qX, 0, 0, M, N).cpu().numpy()
    np.testing.assert_array_equal(I, I_ref)
    if M > 2 and N > 3:  # an interior window
        I2 = lay.group_sums(qX, M // 3, N // 4, M - M // 3, N - N // 4).cpu().numpy()
        np.testing.assert_array_equal(I2, I_ref[:, M // 3:, N // 4:])


@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_forward_matches_oracle(shape):
    M, K, N, r, fmt = shape
    log(f"forward {_ids(shape)}")
    wl = random_layer(M, K, N, r, 7000 + M + K + N, fmt=fmt, x_out=3, w_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    ws = lay.workspace(M)
    Y = lay.forward(to_dev_bf16(wl.X), workspace=ws).cpu().numpy().astype(np.float64)
    Yref = oforward.forward(wl.X, p)["Y"]
    e = rel_err(Y, Yref)
    log(f"  max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y
    if fmt == "int4":
        # the forward path keeps the activation codes in MMA form (FP6 operand words) at
        # the start of its workspace
        codes = decode_mma(ws[:M * K].view(M, K), None, None, "int4", K, 0)[0]
        np.testing.assert_array_equal(codes, oforward.quantize_activations(wl.X, p["inv_s32"], fmt)[1])
    # the two kernels called separately in MMA form, kernel 2 with its split workspace,
    # give the same bits as the forward; without the workspace (no split) the same bar
    X = to_dev_bf16(wl.X)
    qX, sX, la = lay.quantize_act(X, form=svdq.ACT_MMA)
    gws = lay.gemm_workspace(M, svdq.ACT_MMA)
    Y2 = lay.gemm(qX, sX, la, form=svdq.ACT_MMA, workspace=gws).cpu().numpy()
    np.testing.assert_array_equal(Y2, Y.astype(np.float32))
    Yn = lay.gemm(qX, sX, la, form=svdq.ACT_MMA).cpu().numpy().astype(np.float64)
    en = rel_err(Yn, Yref)
    log(f"  unsplit kernel 2 max|err|/RMS = {en:.3e} (split workspace {0 if gws is None else gws.numel()} B)")
    assert en <= TOL_Y
    if K >= 768:
        assert gws is not None, "expected kernel 2 to split this shape"
    # the packed form meets the same bar
    qX, sX, la = lay.quantize_act(X)
    Yp = lay.gemm(qX, sX, la).cpu().numpy().astype(np.float64)
    ep = rel_err(Yp, Yref)
    log(f"  packed form max|err|/RMS = {ep:.3e}")
    assert ep <= TOL_Y


def test_tiny_config_c0():
    wl = make("C0")
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    Y = lay.forward(X).cpu().numpy().astype(np.float64)
    Yref = oforward.forward(wl.X, p)["Y"]
    e = rel_err(Y, Yref)
    log(f"C0 max|err|/RMS = {e:.3e}")
    assert e <= TOL_Y


def test_rank0_and_zero_residual():
    wl = random_layer(200, 256, 300, 8, 99, x_out=3)
    p0 = oracle_pack(wl, rank=0)
    Y = layer_from_oracle(p0).forward(to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
    assert rel_err(Y, oforward.forward(wl.X, p0)["Y"]) <= TOL_Y
    p = dict(oracle_pack(wl))
    p["codesW"] = np.zeros_like(p["codesW"])
    p["qW"] = np.zeros_like(p["qW"])
    Y = layer_from_oracle(p).forward(to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
    ref = oforward.forward(wl.X, p)["Y"]
    assert rel_err(Y, ref) <= 1e-3  # only the low-rank branch remains: fp32-accurate


def test_bf16_output_and_determinism():
    wl = random_layer(257, 256, 300, 8, 5, x_out=3)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    X = to_dev_bf16(wl.X)
    Y32 = lay.forward(X)
    Yb = lay.forward(X, ydtype=svdq.BF16).float().cpu().numpy().astype(np.float64)
    ref = oforward.forward(wl.X, p)["Y"]
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(Yb - ref) <= 2.0 ** -8 * np.abs(ref) + TOL_Y * rms)
    for _ in range(5):
        assert np.array_equal(lay.forward(X).cpu().numpy(), Y32.cpu().numpy())


def test_strided_activation_rows():
    import torch

    wl = random_layer(40, 256, 96, 8, 12, x_out=2)
    p = oracle_pack(wl)
    lay = layer_from_oracle(p)
    Xp = np.zeros((40, 256 + 64), np.uint16)
    Xp[:, :256] = wl.X
    Xd = to_dev_bf16(Xp)[:, :256]
    assert Xd.stride(0) == 320
    Y = lay.forward(Xd).cpu().numpy().astype(np.float64)
    assert rel_err(Y, oforward.forward(wl.X, p)["Y"]) <= TOL_Y


def _ws_lora_region(M, K, rank, fmt):
    """Byte range of lora_act in the forward workspace: MMA-form qX, sX, lora_act in that
    order, each starting on a 256-byte boundary."""
    rup = lambda x: (x + 255) // 256 * 256
    Mp = (M + 3) // 4 * 4
    qx = M * K if fmt == "int4" else (M + 1) // 2 * 2 * (K // 2)
    sx = (K // 64) * Mp * 2 if fmt == "int4" else (K // 32) * Mp
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
    wsf, wsu = lay.workspace(M), lay.workspace(M)
    Yf = lay.forward(X, workspace=wsf).cpu().numpy()
    Yu = lay.forward(X, workspace=wsu, fused=False).cpu().numpy()
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
    Yb = lay.forward(X, ydtype=svdq.BF16, fused=False).float().cpu().numpy().astype(np.float64)
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
    Y = lay.forward(to_dev_bf16(wl.X)).cpu().numpy().astype(np.float64)
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
        Y = Yfull[:, :N]
        lay.forward(Xd, ydtype=ydtype, out=Y, fused=fused)
        assert bool((Yfull[:, N:] == 7.0).all()), "padding columns written"
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
