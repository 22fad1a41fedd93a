"""Oracle: the 4-bit weight-only layer (W4A16), the baseline the method is set against.

Test infrastructure: see the package docstring for who may import this.

Sources (cited by page title and section):
* jeonghoonpark.com "SVDQuant" review, section 3 "Quantization Preliminary", the
  paragraph on why both operands need the same bit width: with 4-bit weights and 16-bit
  activations the weights are upcast to 16 bits before the product, so the product runs
  as a 16-bit one;
* chatpaper.ai SVDQuant abstract: the reported 3.0x speed-up is over a 4-bit
  weight-only quantized baseline.

Readings (the pages give neither the group size, the scale type nor the 16-bit type of
this baseline):
* the weights are quantized by the layer's own INT4 weight quantizer (groups of 64
  along K per output column, fp16 scales max|w| / 7, codes rounded half to even),
  applied to W itself: no smoothing and no low-rank branch (those belong to the
  method, not to the baseline);
* "upcast to 16 bits" is to the activations' type, bf16: each weight becomes
  bf16(s_W q_W), the exact product rounded once to nearest, ties to even;
* the product X Wd is exact here (fp64 sums of exact products); the GPU accumulates in
  fp32.
"""
from __future__ import annotations

import numpy as np

from . import quant
from .numerics import bf16_to_f64, bf16_value_to_bits, f16_to_f64, round_f64_to_bf16


def quantize_weights(W_bits: np.ndarray):
    """W [K][N] (bf16 bits) -> (codes int8 [N][K], fp16 scale bits [K/64][N]): the INT4
    group quantizer per output column n over groups of 64 along K (bf16 values are exact
    in fp32, the quantizer's input type)."""
    Wt = np.ascontiguousarray(bf16_to_f64(W_bits).astype(np.float32).T)  # [N][K]
    codes, sc = quant.quantize_int4(Wt, quant.INT4_GROUP)
    return codes, np.ascontiguousarray(sc.T)


def upcast(codes: np.ndarray, sW_bits: np.ndarray) -> np.ndarray:
    """The 16-bit weights: Wd[k][n] = bf16(s_W[k / 64][n] q[n][k]) as bf16 bits [K][N]
    (the product of an fp16 scale and a code of at most 3 bits is exact in fp64, then one
    rounding to bf16, nearest, ties to even)."""
    N, K = codes.shape
    s = f16_to_f64(sW_bits)  # [K/64][N]
    prod = codes.T.astype(np.float64) * np.repeat(s, quant.INT4_GROUP, axis=0)[:K]
    return bf16_value_to_bits(round_f64_to_bf16(prod))


def forward(X_bits: np.ndarray, codes: np.ndarray, sW_bits: np.ndarray, rows=None, cols=None) -> np.ndarray:
    """Y = X Wd in fp64 (X bf16 bits [M][K]); rows / cols select a sub-block of Y."""
    Wd = bf16_to_f64(upcast(codes, sW_bits))
    X = bf16_to_f64(X_bits)
    if rows is not None:
        X = X[rows]
    if cols is not None:
        Wd = Wd[:, cols]
    return X @ Wd
