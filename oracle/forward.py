"""Oracle: the layer's forward pass, step by step.

Test infrastructure: see the package docstring for who may import this.

Y = Q(X_hat) Q(R) + (X_hat L1) L2,  X_hat = X diag(s)^-1
(jeonghoonpark.com "SVDQuant" review, section 4.2, the decomposition equation; the
scaled low-bit product s_X s_W Q_X Q_W of section 3, applied per K-group).

Steps, in the order the fused kernels of section 4.3 ("Nunchaku") take them:
  1. smooth X (runtime half of the smoothing equation),
  2. per-group absmax, scale, 4-bit codes of X_hat,
  3. low-rank down projection X_hat L1 (fused with 1-2 on the GPU),
  4. integer group sums of the 4-bit codes,
  5. per-group rescale by s_X s_W and sum over groups,
  6. low-rank up projection added to the result (fused with 4-5 on the GPU).
All arithmetic is fp64 (exact for 1-4) or exact integers.
"""
from __future__ import annotations

import numpy as np

from . import quant
from .numerics import f16_to_f64


def quantize_activations(X_bits: np.ndarray, inv_s32: np.ndarray, fmt: str, S_X=None):
    """Steps 1-2.  Returns (X_hat fp32 [M][K], codes [M][K], scales [M][K/G]); NVFP4
    quantizes under the activations' tensor scale S_X."""
    Xh = quant.smooth_activations(X_bits, inv_s32)
    if fmt == "int4":
        codes, sc = quant.quantize_int4(Xh, quant.INT4_GROUP)
    elif fmt == "mxfp4":
        codes, sc = quant.quantize_mxfp4(Xh, quant.FP4_GROUP)
    elif fmt == "nvfp4":
        codes, sc = quant.quantize_nvfp4(Xh, S_X)
    else:
        raise ValueError(fmt)
    return Xh, codes, sc


def lora_down(Xh32: np.ndarray, L1b: np.ndarray) -> np.ndarray:
    """Step 3: X_hat L1 in fp64 (fp32 and bf16 inputs are exact in fp64)."""
    return np.asarray(Xh32, dtype=np.float64) @ np.asarray(L1b, dtype=np.float64)


def group_sums(cX: np.ndarray, cW: np.ndarray, G: int) -> np.ndarray:
    """Step 4 (INT4): I[g, m, n] = sum over k in group g of qX[m,k] qW[n,k].

    cX [M][K], cW [N][K] integer codes.  Each block product is an fp64 matmul of
    integer-valued matrices whose partial sums stay far below 2^53, hence exact.
    """
    M, K = cX.shape
    out = np.empty((K // G, M, cW.shape[0]), dtype=np.int64)
    for g in range(K // G):
        a = cX[:, g * G:(g + 1) * G].astype(np.float64)
        b = cW[:, g * G:(g + 1) * G].astype(np.float64)
        out[g] = np.rint(a @ b.T).astype(np.int64)
    return out


def code_product(cX: np.ndarray, cW: np.ndarray) -> np.ndarray:
    """Sum over all groups of the integer group sums: the plain integer product of the
    codes, sum_k qX[m,k] qW[n,k] (cX [M][K], cW [N][K]).  One fp64 matmul of
    integer-valued matrices; every partial sum is far below 2^53, so it is exact.
    This is what the 4-bit product of section 3 reduces to when every scale is 1."""
    return np.rint(cX.astype(np.float64) @ cW.astype(np.float64).T).astype(np.int64)


def residual_int4(cX, sX_bits, cW, sW_bits, rows=None, cols=None) -> np.ndarray:
    """Steps 4-5 (INT4): sum_g s_X[m,g] s_W[g,n] I[g,m,n] in fp64.

    cX [M][K] int codes, sX_bits [M][K/64] fp16 bits; cW [N][K], sW_bits [K/64][N].
    rows / cols select a subset of outputs (index arrays), for sampled checks.
    """
    G = quant.INT4_GROUP
    if rows is not None:
        cX, sX_bits = cX[rows], sX_bits[rows]
    if cols is not None:
        cW, sW_bits = cW[cols], sW_bits[:, cols]
    sX = f16_to_f64(sX_bits)
    sW = f16_to_f64(sW_bits)
    M, K = cX.shape
    Y = np.zeros((M, cW.shape[0]))
    for g in range(K // G):
        a = cX[:, g * G:(g + 1) * G].astype(np.float64)
        b = cW[:, g * G:(g + 1) * G].astype(np.float64)
        Ig = a @ b.T  # exact integers
        Y += (sX[:, g][:, None] * sW[g][None, :]) * Ig
    return Y


def residual_mxfp4(cX, eX, cW, eW, rows=None, cols=None) -> np.ndarray:
    """Steps 4-5 (FP4): sum_g 2^(eX[m,g] + eW[g,n]) sum_k vX vW in fp64.

    cX [M][K] E2M1 codes, eX [M][K/32] E8M0 bytes; cW [N][K], eW [K/32][N].
    Each group's dot product of E2M1 values is exact in fp64.
    """
    G = quant.FP4_GROUP
    if rows is not None:
        cX, eX = cX[rows], eX[rows]
    if cols is not None:
        cW, eW = cW[cols], eW[:, cols]
    vX = quant.e2m1_value(cX)
    vW = quant.e2m1_value(cW)
    sX = np.ldexp(1.0, eX.astype(np.int32) - 127)
    sW = np.ldexp(1.0, eW.astype(np.int32) - 127)
    M, K = cX.shape
    Y = np.zeros((M, cW.shape[0]))
    for g in range(K // G):
        Pg = vX[:, g * G:(g + 1) * G] @ vW[:, g * G:(g + 1) * G].T
        Y += (sX[:, g][:, None] * sW[g][None, :]) * Pg
    return Y


def residual_nvfp4(cX, eX, S_X, cW, eW, S_W, rows=None, cols=None) -> np.ndarray:
    """Steps 4-5 (NVFP4-style): S_X S_W sum_g sX[m,g] sW[g,n] sum_k vX vW in fp64.

    cX [M][K] E2M1 codes, eX [M][K/16] E4M3 bytes; cW [N][K], eW [K/16][N]; S_X, S_W the
    fp32 tensor scales.  Each group's dot product of E2M1 values is exact in fp64."""
    G = quant.NV_GROUP
    if rows is not None:
        cX, eX = cX[rows], eX[rows]
    if cols is not None:
        cW, eW = cW[cols], eW[:, cols]
    vX = quant.e2m1_value(cX)
    vW = quant.e2m1_value(cW)
    sX = quant.e4m3_value(eX)
    sW = quant.e4m3_value(eW)
    M, K = cX.shape
    Y = np.zeros((M, cW.shape[0]))
    for g in range(K // G):
        Pg = vX[:, g * G:(g + 1) * G] @ vW[:, g * G:(g + 1) * G].T
        Y += (sX[:, g][:, None] * sW[g][None, :]) * Pg
    return Y * (np.float64(np.float32(S_X)) * np.float64(np.float32(S_W)))


def forward(X_bits: np.ndarray, packed: dict, rows=None, cols=None) -> dict:
    """Full layer.  ``packed`` holds inv_s32, L1b [K][r], L2b [r][N], codesW [N][K],
    sW [K/G][N] and fmt (as produced by oracle.pack, or the same arrays from elsewhere).

    Returns dict(Xh, codesX, scalesX [M][K/G], lora_act [M][r], Y [rows][cols]).
    """
    fmt = packed["fmt"]
    Xh, cX, sX = quantize_activations(X_bits, packed["inv_s32"], fmt, packed.get("S_X"))
    la = lora_down(Xh, packed["L1b"]) if packed["L1b"].shape[1] else np.zeros((Xh.shape[0], 0))
    if fmt == "int4":
        Y = residual_int4(cX, sX, packed["codesW"], packed["sW"], rows, cols)
    elif fmt == "nvfp4":
        Y = residual_nvfp4(cX, sX, packed["S_X"], packed["codesW"], packed["sW"], packed["S_W"], rows, cols)
    else:
        Y = residual_mxfp4(cX, sX, packed["codesW"], packed["sW"], rows, cols)
    la_r = la if rows is None else la[rows]
    L2 = np.asarray(packed["L2b"], dtype=np.float64)
    L2c = L2 if cols is None else L2[:, cols]
    if L2.shape[0]:
        Y = Y + la_r @ L2c
    return dict(Xh=Xh, codesX=cX, scalesX=sX, lora_act=la, Y=Y)


# ---------------------------------------------------------------------------------------
# The chained MLP pair: fc2 consumes GELU of fc1's output.  The fusion that motivates
# chaining the pair (the next layer's quantization done where the previous layer's output
# tile is produced, so the 16-bit activation is not written and re-read) is the fused
# kernel design of the review's section 4.3 ("Nunchaku", Figure 6(b)) and the cost named
# in the ch3chohch3 post's "量化方案" section (16-bit activations reloaded from HBM).
# Readings (the pages name neither the activation nor the hidden format):
#   * the activation is GELU in its exact form x Phi(x), Phi the standard normal CDF;
#   * the hidden activation G exists in the layers' 16-bit input format: one rounding of
#     GELU(H) to bf16 (ties to even), H = fc1's output;
#   * fc2 is the unchanged layer forward above, applied to G.

def gelu_erf(h: np.ndarray) -> np.ndarray:
    """GELU(h) = h Phi(h) with Phi(h) = erfc(-h / sqrt 2) / 2, in fp64 (erfc rather than
    1 + erf keeps full relative accuracy in the negative tail)."""
    from scipy.special import erfc

    h = np.asarray(h, dtype=np.float64)
    return h * (0.5 * erfc(-h / np.sqrt(2.0)))


def mlp_hidden(X_bits: np.ndarray, packed1: dict) -> dict:
    """fc1's forward, then G = bf16(GELU(H)).  Returns dict(H [M][N1] fp64, G_bits uint16
    [M][N1], fc1 = fc1's forward dict)."""
    from .numerics import bf16_value_to_bits, round_f64_to_bf16

    f1 = forward(X_bits, packed1)
    H = f1["Y"]
    G_bits = bf16_value_to_bits(round_f64_to_bf16(gelu_erf(H)))
    return dict(H=H, G_bits=G_bits, fc1=f1)


def mlp_forward(X_bits: np.ndarray, packed1: dict, packed2: dict, cols=None) -> dict:
    """The pair: Y = fc2(bf16(GELU(fc1(X)))).  Every token is independent, so a subset of
    tokens is taken by passing those rows of X; cols selects fc2's output columns.
    Returns dict(H, G_bits, fc2 = fc2's forward dict (its Y is the pair's output))."""
    hid = mlp_hidden(X_bits, packed1)
    f2 = forward(hid["G_bits"], packed2, cols=cols)
    return dict(H=hid["H"], G_bits=hid["G_bits"], fc2=f2)
