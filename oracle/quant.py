"""Oracle: smoothing and the two 4-bit group quantizers.

Test infrastructure: see the package docstring for who may import this.

Sources (cited by page title and section):
* smoothing equation Y = (X diag(s)^-1)(diag(s) W) and the factor
  s_j = max|X_j|^alpha / max|W_j|^(1-alpha): ch3chohch3.github.io, "从 Smooth Quant 到
  SVD Quant", section "Smooth Quant（W8A8）", the two displayed equations;
* quantizer Q_X = round(X / s_X), s_X = max|X| / q_max, q_max = 6 for 4-bit float:
  jeonghoonpark.com "SVDQuant" review, section 3 "Quantization Preliminary", first
  displayed equation and the line after it.  q_max = 7 for INT4, group sizes (64 for
  INT4 with fp16 scales, 32 for FP4 with power-of-two E8M0 scales) are the workloads'
  choices; the pages only give the per-tensor formula.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import bf16_to_f64

INT4_QMAX = 7
FP4_QMAX = 6.0
INT4_GROUP = 64
FP4_GROUP = 32
# E2M1 magnitudes, indexed by the 3 low bits of the code (exponent:mantissa)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FP16_MAX = 65504.0
SMOOTH_FLOOR = 1e-5


def smoothing_factors(act_absmax, w_absmax, alpha: float):
    """Per-input-channel smoothing factor s_j = max|X_j|^a / max|W_j|^(1-a).

    Readings taken where the page is silent:
    * "channel j" of W is row j of W [K x N] (the side diag(s) multiplies);
    * a zero maximum is floored at 1e-5 so that s stays finite and non-zero;
    * s is evaluated in fp64 with the C library's scalar ``pow`` (math.pow), the
      exponent 1-a taken in fp64; it is stored as fp32 (s32), and the runtime
      multiplies by inv_s32 = fp32(1 / s32) (IEEE single division).
    Returns (s64, s32, inv_s32).
    """
    a = np.maximum(np.asarray(act_absmax, dtype=np.float64), SMOOTH_FLOOR)
    w = np.maximum(np.asarray(w_absmax, dtype=np.float64), SMOOTH_FLOOR)
    beta = 1.0 - float(alpha)
    s64 = np.array([math.pow(float(ai), float(alpha)) / math.pow(float(wi), beta)
                    for ai, wi in zip(a, w)], dtype=np.float64)
    s32 = s64.astype(np.float32)
    inv_s32 = np.float32(1.0) / s32
    return s64, s32, inv_s32


def channel_absmax_rows(M_bits: np.ndarray) -> np.ndarray:
    """max over the columns of |M| for each row (bf16 input, exact)."""
    return np.abs(bf16_to_f64(M_bits)).max(axis=1)


def channel_absmax_cols(M_bits: np.ndarray) -> np.ndarray:
    """max over the rows of |M| for each column (bf16 input, exact)."""
    return np.abs(bf16_to_f64(M_bits)).max(axis=0)


def smooth_activations(X_bits: np.ndarray, inv_s32: np.ndarray) -> np.ndarray:
    """X_hat = X * diag(s)^-1, one fp32 product per element (RNE).

    The product of a bf16 value and an fp32 value is exact in fp64; casting it to fp32
    is the single rounding an fp32 multiply performs.
    """
    x = bf16_to_f64(X_bits)
    return (x * np.asarray(inv_s32, dtype=np.float64)[None, :]).astype(np.float32)


def _groups(v: np.ndarray, G: int) -> np.ndarray:
    v = np.asarray(v)
    assert v.shape[-1] % G == 0, "K must be a multiple of the group size"
    return v.reshape(v.shape[:-1] + (v.shape[-1] // G, G))


def int4_scale(absmax32: np.ndarray) -> np.ndarray:
    """s = max|v| / q_max as fp32 (IEEE division), stored as fp16 (RNE), saturating.

    Returns fp16 bit patterns.  fp16 overflow saturates to the largest finite fp16.
    """
    a = np.asarray(absmax32, dtype=np.float32)
    s32 = a / np.float32(INT4_QMAX)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    s16 = np.where(np.isinf(s16), np.float16(FP16_MAX), s16)
    return s16.view(np.uint16)


def quantize_int4(v32: np.ndarray, G: int = INT4_GROUP):
    """Symmetric INT4 quantization of fp32 values in groups of G along the last axis.

    Per group: a = max|v|; s = fp16(fp32(a / 7)); q = round(v / s) with the exact real
    quotient rounded half to even, clamped to [-7, 7]; a group whose fp16 scale is 0
    gets all-zero codes.

    Exactness of the rounding decision: v (24-bit significand) / s (11-bit) is formed
    in fp64.  If v/s is not a half-integer, its distance to the nearest half-integer
    is at least 2^-27 whenever v/s >= 1/2, far above the fp64 rounding error, so
    rint(fp64(v/s)) equals round-half-even of the exact quotient.

    Returns (codes int8 [..., K], scale fp16 bits uint16 [..., K/G]).
    """
    g = _groups(np.asarray(v32, dtype=np.float32), G)
    a = np.abs(g).max(axis=-1)
    sbits = int4_scale(a)
    s = sbits.view(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = g.astype(np.float64) / s[..., None]
    q = np.rint(t)
    q = np.clip(q, -INT4_QMAX, INT4_QMAX)
    q = np.where((s == 0)[..., None], 0.0, q)
    codes = q.astype(np.int8).reshape(np.asarray(v32).shape)
    return codes, sbits


def dequant_int4(codes: np.ndarray, sbits: np.ndarray, G: int = INT4_GROUP) -> np.ndarray:
    """s * q per element (fp64)."""
    s = sbits.view(np.float16).astype(np.float64)
    g = _groups(codes.astype(np.float64), G) * s[..., None]
    return g.reshape(codes.shape)


def fp4_exponent(absmax32: np.ndarray) -> np.ndarray:
    """Shared power-of-two exponent e of an FP4 group: the smallest e with 6*2^e >= a.

    Reading: the page's s = max|v| / q_max (q_max = 6) must be a power of two in the
    E8M0 format, and it is rounded *up*, so |v / 2^e| <= 6 and nothing saturates.
    With a = m * 2^E, m in [1, 2): e = E - 2 if m <= 1.5, else E - 1.  An all-zero
    group gets e = 0.  e is clamped to the E8M0 range [-127, 127].
    """
    a = np.asarray(absmax32, dtype=np.float64)
    f, E = np.frexp(a)  # a = f * 2^E, f in [0.5, 1)
    m = 2.0 * f
    Eb = E - 1
    e = np.where(m <= 1.5, Eb - 2, Eb - 1)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int32)


def e2m1_round(u: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude index for |u| <= 6, ties to the even index.

    The index's lowest bit is the E2M1 mantissa bit, so "even index" is round half
    to even on the format's own grid {0, .5, 1, 1.5, 2, 3, 4, 6}.
    """
    u = np.abs(np.asarray(u, dtype=np.float64))
    d = np.abs(u[..., None] - E2M1_GRID)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # first even candidate if any, else the (unique) odd one
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    return idx.astype(np.uint8)


def quantize_mxfp4(v32: np.ndarray, G: int = FP4_GROUP):
    """FP4 (E2M1) quantization with one E8M0 power-of-two scale per group of G.

    code = (sign bit of v) << 3 | index of round(v / 2^e) on the E2M1 grid.
    The sign bit is kept for values that round to zero (so -0.0 and small negative
    values give code 0x8); scaling by 2^-e is exact.
    Returns (codes uint8 [..., K] in 0..15, e8m0 bytes uint8 [..., K/G]).
    """
    v = np.asarray(v32, dtype=np.float32)
    g = _groups(v, G)
    a = np.abs(g).max(axis=-1).astype(np.float64)
    e = fp4_exponent(a)
    u = np.ldexp(g.astype(np.float64), -e[..., None])
    idx = e2m1_round(u)
    sign = np.signbit(g).astype(np.uint8)
    codes = ((sign << 3) | idx).reshape(v.shape).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """E2M1 code -> value (fp64)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_GRID[c & 7]
    return np.where(c & 8, -mag, mag)


def dequant_mxfp4(codes: np.ndarray, e8m0: np.ndarray, G: int = FP4_GROUP) -> np.ndarray:
    e = e8m0.astype(np.int32) - 127
    g = _groups(e2m1_value(codes), G) * np.ldexp(1.0, e)[..., None]
    return g.reshape(codes.shape)


def int4_to_nibble(q: np.ndarray) -> np.ndarray:
    """INT4 code q in [-7, 7] -> 4-bit sign-magnitude nibble (bit 3 sign, bits 0-2 |q|).

    Reading: the pages fix no bit encoding.  Sign-magnitude is the layout E2M1 codes
    already use (sign in bit 3), and zero is always 0x0.
    """
    q = np.asarray(q).astype(np.int16)
    return (((q < 0).astype(np.uint8) << 3) | np.abs(q).astype(np.uint8)).astype(np.uint8)


def nibble_to_int4(n: np.ndarray) -> np.ndarray:
    n = np.asarray(n, dtype=np.uint8)
    mag = (n & 7).astype(np.int8)
    return np.where(n & 8, -mag, mag).astype(np.int8)


def pack_nibbles(nibbles: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte along the last axis: byte j = n[2j] | n[2j+1] << 4."""
    c = (np.asarray(nibbles).astype(np.uint16) & 0xF).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles: 4-bit codes (uint8, 0..15)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- NVFP4-style (group 16)
# The ch3chohch3.github.io post "从 Smooth Quant 到 SVD Quant", section "个人见解",
# discusses SVDQuant under nvfp4, "a group-16 two-level-scale scheme", and reports a
# relative-error gain of 1.16-3x over bare nvfp4.  The page defines the format no further;
# the readings taken here:
# * codes: E2M1, as for FP4 above (sign bit kept, round half to even on the grid);
# * level 1: one FP8 E4M3 scale per 16 consecutive values along K (4 exponent bits, bias
#   7, 3 mantissa bits, subnormals down to 2^-9, largest finite 448), rounded to nearest
#   even and saturating at 448;
# * level 2: one fp32 scale per tensor, S = fp32(amax / 2688) with 2688 = 6 * 448 (the
#   largest E2M1 magnitude times the largest E4M3 value), amax the tensor's max |v|
#   (weights: the residual; activations: the smoothed calibration activations, fixed
#   offline like the smoothing factor); S = 1 for an all-zero tensor;
# * the group scale is s = E4M3(fp32(a * r6)) with a = max|v| of the group and r6 =
#   fp32(1 / fp32(6 S)), the code is E2M1(fp32(v * fp32(1 / sigma))) with sigma =
#   fp32(s * S) (the page's Q = round(X / s) taken as a multiply by the fp32 reciprocal),
#   saturating at 6; a group whose E4M3 scale is 0 gets sign-kept zero codes.
# Dequantized value: S * s * e2m1(code).
NV_GROUP = 16
E4M3_MAX = 448.0
NV_TSCALE_DIV = 6.0 * E4M3_MAX


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest FP8 E4M3 value of non-negative x (ties to the even mantissa), saturating
    at 448.  Normal values (1 + m/8) 2^(E-7), E in 1..15 (E = 15 stops at m = 6);
    subnormals m 2^-9.  The quantum of a value with binary exponent e is
    2^(max(e, -6) - 3); the value is divided by it (exact), rounded with rint, scaled back."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x > 0
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    out[nz] = np.rint(x[nz] / q) * q
    return np.minimum(out, E4M3_MAX)


def e4m3_bits(v: np.ndarray) -> np.ndarray:
    """Non-negative E4M3 values (as produced by e4m3_round) -> bytes."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, np.uint8)
    nz = v > 0
    m, e = np.frexp(v[nz])  # v = m 2^e, m in [0.5, 1)
    E = e - 1 + 7  # biased exponent of a normal value
    sub = E < 1
    mant = np.where(sub, np.rint(v[nz] / 2.0 ** -9), np.rint((2 * m - 1) * 8)).astype(np.int64)
    out[nz] = np.where(sub, mant, (E.astype(np.int64) << 3) | mant).astype(np.uint8)
    return out


def e4m3_value(b: np.ndarray) -> np.ndarray:
    """E4M3 bytes (sign bit 0) -> values."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    E, m = (b >> 3) & 15, b & 7
    return np.where(E == 0, m * 2.0 ** -9, (1 + m / 8.0) * np.ldexp(1.0, E - 7))


def nvfp4_tensor_scale(amax) -> np.float32:
    """Level-2 scale S = fp32(amax / 2688) (IEEE fp32 division), 1 for amax = 0."""
    a = np.float32(amax)
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(NV_TSCALE_DIV))


def quantize_nvfp4(v32: np.ndarray, S: np.float32):
    """Group-16 E2M1 codes with E4M3 group scales under the fp32 tensor scale S.
    Returns (codes uint8 [..., K] in 0..15, E4M3 bytes uint8 [..., K/16])."""
    v = np.asarray(v32, dtype=np.float32)
    g = _groups(v, NV_GROUP)
    S = np.float32(S)
    r6 = np.float32(1.0) / np.float32(np.float32(6.0) * S)
    a = np.abs(g).max(axis=-1)
    s = e4m3_round((a * r6).astype(np.float32))  # level-1 scale values
    sigma = (s.astype(np.float32) * S).astype(np.float32)
    with np.errstate(divide="ignore"):
        rcp = np.where(sigma > 0, np.float32(1.0) / np.where(sigma > 0, sigma, 1), np.float32(0.0)).astype(np.float32)
    t = (g * rcp[..., None]).astype(np.float32)  # one fp32 rounding
    idx = e2m1_round(np.minimum(np.abs(t.astype(np.float64)), 6.0))
    sign = np.signbit(g).astype(np.uint8)
    codes = ((sign << 3) | idx).reshape(v.shape).astype(np.uint8)
    return codes, e4m3_bits(s)


def dequant_nvfp4(codes: np.ndarray, e4m3: np.ndarray, S) -> np.ndarray:
    g = _groups(e2m1_value(codes), NV_GROUP) * e4m3_value(e4m3)[..., None] * np.float64(np.float32(S))
    return g.reshape(codes.shape)
