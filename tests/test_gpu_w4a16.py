"""GPU parity of the 4-bit weight-only baseline (svdq_w4a16_gemm) against the oracle.

The weights are W's own INT4 codes and fp16 group scales from the oracle's quantizer,
uploaded as the layer; where the library's host quantizer applies (K a multiple of 128)
its codes and scales must be the oracle's, bit for bit.  Y is compared
element by element with the oracle's exact product X bf16(s q) under the fp32
accumulation bound |Y - Y_ref| <= gamma_K (|X| |Wd|), gamma_K = K u / (1 - K u) with u =
2^-23 (any order of K fp32 additions, rounding or truncating), plus half a bf16 step of
the result for bf16 output.  Outputs are pre-filled with NaN, so an unwritten element
fails, and the padding of a strided output must keep its sentinel.
"""
import numpy as np
import pytest

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import make, random_layer
from gpu_helpers import log, to_dev_bf16
from oracle import pack as opack, weight_only as owo
from oracle.numerics import bf16_to_f64

pytestmark = pytest.mark.gpu

SHAPES = [  # M, K, N: ragged M and N (one to three tiles each way), odd and even stage counts
    (1, 64, 1), (5, 128, 7), (33, 192, 130), (257, 320, 129), (300, 512, 256), (600, 1024, 384),
]


def _bound(X_bits, Wd_bits, K, ref, bf16_out):
    u = 2.0 ** -23
    gam = K * u / (1 - K * u)
    A = np.abs(bf16_to_f64(X_bits)) @ np.abs(bf16_to_f64(Wd_bits))
    b = gam * A
    if bf16_out:
        b = b + 2.0 ** -8 * (np.abs(ref) + b)
    return b + 1e-30


def _run(lay, X_bits, ydtype, ldx_pad=0, ldy_pad=0):
    import torch

    M, K = X_bits.shape
    Xp = np.zeros((M, K + ldx_pad), np.uint16)
    Xp[:, :K] = X_bits
    X = to_dev_bf16(Xp)[:, :K]
    dt = torch.float32 if ydtype == svdq.F32 else torch.bfloat16
    Yfull = torch.full((M, lay.N + ldy_pad), float("nan"), dtype=dt, device="cuda:0")
    Y = Yfull[:, : lay.N]
    lay.forward(X, ydtype, out=Y)
    torch.cuda.synchronize()
    Yf = Yfull.float().cpu().numpy().astype(np.float64)
    if ldy_pad:
        assert np.isnan(Yf[:, lay.N:]).all(), "padding of Y written"
    return Yf[:, : lay.N]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("ydtype", [svdq.F32, svdq.BF16])
def test_w4a16_matches_oracle(shape, ydtype):
    M, K, N = shape
    log(f"[w4a16] M={M} K={K} N={N} ydtype={ydtype}")
    wl = random_layer(M, K, N, 0, seed=700 + M + K + N)
    codes, sW = owo.quantize_weights(wl.W)
    lay = svdq.WeightOnlyLinear(K, N, opack.pack_codes(codes, "int4"), sW)
    if K % 128 == 0:
        # the library's host quantizer gives the oracle's codes and scales
        lib = svdq.WeightOnlyLinear.from_weights(wl.W)
        np.testing.assert_array_equal(lib.qW.cpu().numpy(), lay.qW.cpu().numpy())
        np.testing.assert_array_equal(lib.sW.cpu().numpy(), lay.sW.cpu().numpy())
    pad = (8, 3) if M > 5 else (0, 0)
    Y = _run(lay, wl.X, ydtype, *pad)
    ref = owo.forward(wl.X, codes, sW)
    assert np.isfinite(Y).all(), "unwritten or non-finite outputs"
    bound = _bound(wl.X, owo.upcast(codes, sW), K, ref, ydtype == svdq.BF16)
    err = np.abs(Y - ref)
    assert (err <= bound).all(), f"max err/bound {np.max(err / bound):.3g}"


def test_w4a16_full_size_qkv_every_element():
    """The FLUX.1 QKV shape (4608 x 3072 -> 9216), the bench's launch, every element."""
    wl = make("C1")
    log(f"[w4a16] full size M={wl.M} K={wl.K} N={wl.N}")
    codes, sW = owo.quantize_weights(wl.W)
    lay = svdq.WeightOnlyLinear.from_weights(wl.W)
    Y = _run(lay, wl.X, svdq.F32)
    ref = owo.forward(wl.X, codes, sW)
    assert np.isfinite(Y).all()
    bound = _bound(wl.X, owo.upcast(codes, sW), wl.K, ref, False)
    err = np.abs(Y - ref)
    log(f"[w4a16] max err/bound {np.max(err / bound):.3g}, max err/RMS {err.max() / np.sqrt(np.mean(ref ** 2)):.3g}")
    assert (err <= bound).all()


def test_w4a16_deterministic():
    import torch

    wl = random_layer(700, 512, 384, 0, seed=77)
    lay = svdq.WeightOnlyLinear.from_weights(wl.W)
    X = to_dev_bf16(wl.X)
    a = lay.forward(X).cpu()
    b = lay.forward(X).cpu()
    assert torch.equal(a, b)


def test_w4a16_planted_scales_and_codes():
    """Codes and scales set directly: every code -7..7 and the negative-zero nibble, scales
    0, the smallest fp16 subnormal, the largest subnormal, 1 and the saturated 65504, and
    scale products that are bf16 ties; X with magnitudes that keep every product finite."""
    import torch

    rng = np.random.default_rng(21)
    M, K, N = 70, 384, 136
    codes = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    nib = (np.where(codes < 0, 8, 0) | np.abs(codes)).astype(np.uint8)
    zero = codes == 0
    nib[zero & (rng.random((N, K)) < 0.5)] = 8  # -0: sign bit with magnitude 0
    qW = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    special = np.array([0x0000, 0x0001, 0x03FF, 0x3C00, 0x7BFF, 0x3C04, 0x3C0C, 0x3C02], np.uint16)
    sW = rng.integers(0x2000, 0x4800, size=(K // 64, N)).astype(np.uint16)
    sW.flat[:: 5] = special[np.arange(sW.size)[:: 5] % special.size]
    X = (rng.standard_normal((M, K)) * 0.5).astype(np.float32)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)  # truncated to bf16: any bf16 input
    lay = svdq.WeightOnlyLinear(K, N, qW, sW)
    Y = _run(lay, Xb, svdq.F32, 8, 4)
    ref = owo.forward(Xb, codes, sW)
    assert np.isfinite(Y).all()
    bound = _bound(Xb, owo.upcast(codes, sW), K, ref, False)
    err = np.abs(Y - ref)
    assert (err <= bound).all(), f"max err/bound {np.max(err / bound):.3g}"
