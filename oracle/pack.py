"""Oracle: offline weight packing (smoothing, SVD split, residual quantization) and
the LoRA fold.

Test infrastructure: see the package docstring for who may import this.

Sources:
* weight side of smoothing, W_hat = diag(s) W: ch3chohch3.github.io "从 Smooth Quant
  到 SVD Quant", section "Smooth Quant（W8A8）", first displayed equation;
* SVD split W_hat = L1 L2 + R with L1 = U Sigma_r, L2 = V_r^T, rank 32 by default,
  L1 [hidden x r], L2 [r x hidden], low-rank branch kept in 16 bit and only R
  quantized to 4 bit: jeonghoonpark.com "SVDQuant" review, section 4.2, the bullet
  list defining L1, L2, R and the decomposition equation; the same post on
  ch3chohch3.github.io, section "量化方案", the truncation equation;
* static artifacts (weight scales, smoothing factor, low-rank branch) fixed offline:
  ch3chohch3.github.io post, section "量化方案", item 1;
* LoRA adapters used without re-quantizing R: SVDQuant abstract (chatpaper.ai);
* R optimised repeatedly rather than from a single split: jeonghoonpark.com "SVDQuant"
  review, the discussion after "Limitation", item on accuracy (refine_split).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64, round_f64_to_bf16, bf16_value_to_bits
from . import quant


def smoothed_weight(W_bits: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """W_hat = diag(s) W in fp64 (a bf16 times an fp32 value is exact in fp64)."""
    return np.asarray(s32, dtype=np.float64)[:, None] * bf16_to_f64(W_bits)


def svd_split(W_hat: np.ndarray, rank: int):
    """Truncated SVD split of the smoothed weight.

    L1 = U_r Sigma_r (the page writes U Sigma_r; U_r, the first r columns, is the
    reading), L2 = V_r^T.  Both factors are rounded to bf16 (RNE, one rounding from
    fp64), and R absorbs that rounding: R = W_hat - L1b L2b in fp64, so
    W_hat = L1b L2b + R holds with the stored factors.  Sigma goes entirely into L1.
    The SVD is LAPACK's (numpy.linalg.svd), a library step.
    Returns dict(L1, L2 unrounded; L1b, L2b bf16 values; R fp64; sigma).
    """
    U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
    L1 = U[:, :rank] * S[:rank]
    L2 = Vt[:rank, :]
    L1b = round_f64_to_bf16(L1)
    L2b = round_f64_to_bf16(L2)
    R = W_hat - L1b @ L2b
    return dict(L1=L1, L2=L2, L1b=L1b, L2b=L2b, R=R, sigma=S)


def residual_tensor_scale(R32: np.ndarray) -> np.float32:
    """NVFP4-style level-2 scale of the residual: from its max |R| over the whole tensor."""
    return quant.nvfp4_tensor_scale(np.abs(np.asarray(R32, dtype=np.float32)).max())


def quantize_residual(R32: np.ndarray, fmt: str):
    """Quantize R [K x N] per output column n, in groups along K.

    Returns (codes [N][K], scales [K/G][N]): INT4 codes int8 with fp16 scale bits, or
    E2M1 codes uint8 with E8M0 bytes (MXFP4) or E4M3 bytes (NVFP4, under the tensor scale
    residual_tensor_scale(R32)).
    """
    Rt = np.ascontiguousarray(np.asarray(R32, dtype=np.float32).T)  # [N][K]
    if fmt == "int4":
        codes, sc = quant.quantize_int4(Rt, quant.INT4_GROUP)
    elif fmt == "mxfp4":
        codes, sc = quant.quantize_mxfp4(Rt, quant.FP4_GROUP)
    elif fmt == "nvfp4":
        codes, sc = quant.quantize_nvfp4(Rt, residual_tensor_scale(R32))
    else:
        raise ValueError(fmt)
    return codes, np.ascontiguousarray(sc.T)


def dequant_residual(codes: np.ndarray, sW: np.ndarray, fmt: str, S=None) -> np.ndarray:
    """deq(Q(R)) [K][N] in fp64 from codes [N][K] and group-major scales [K/G][N]
    (NVFP4: S is the tensor scale the codes were made under)."""
    sc = np.ascontiguousarray(np.asarray(sW).T)  # [N][K/G]
    if fmt == "int4":
        D = quant.dequant_int4(codes, sc, quant.INT4_GROUP)
    elif fmt == "mxfp4":
        D = quant.dequant_mxfp4(codes, sc, quant.FP4_GROUP)
    elif fmt == "nvfp4":
        D = quant.dequant_nvfp4(codes, sc, S)
    else:
        raise ValueError(fmt)
    return np.ascontiguousarray(D.T)


def split_error(W_hat: np.ndarray, L1b: np.ndarray, L2b: np.ndarray, fmt: str):
    """The split's weight error with the stored factors and the quantized residual:
    R = W_hat - L1b L2b (fp64), codes and scales of fp32(R), and
    E = ||W_hat - L1b L2b - deq(Q(R))||_F (the quantization error of the decomposition,
    review section 4.1 measures errors in the Frobenius norm)."""
    R = W_hat - L1b @ L2b
    R32 = R.astype(np.float32)
    codes, sW = quantize_residual(R32, fmt)
    D = dequant_residual(codes, sW, fmt, residual_tensor_scale(R32) if fmt == "nvfp4" else None)
    return dict(R=R, codes=codes, sW=sW, D=D, err=float(np.linalg.norm(R - D)))


def refine_split(W_hat: np.ndarray, rank: int, fmt: str, iters: int, keep_iterates: bool = False):
    """Iterative refinement of the split (jeonghoonpark.com "SVDQuant" review, the
    discussion after "Limitation", item on accuracy: the low-rank split is not taken
    once, R is optimised repeatedly to reduce the quantization error).

    Reading (the page names no algorithm): alternate between the residual's quantized
    value and the low-rank factors.  Iterate 0 is the plain split of svd_split.  Iterate
    t >= 1 takes the rank-r split of W_hat - deq(Q(R_{t-1})) (the part of W_hat the
    quantized residual does not already carry), rounds its factors to bf16 and sets
    R_t = W_hat - L1b L2b, so W_hat = L1b L2b + R_t still holds exactly.  Each iterate's
    error is split_error's E; the iterate with the smallest E is kept (the first on
    ties), so refinement never returns a worse pack than the plain split.

    Returns (best: dict with L1, L2, L1b, L2b, R, codes, sW, err; errors: list of the
    iters + 1 iterates' E; index of the best iterate).  keep_iterates: best["iterates"]
    lists every iterate's target and factors.
    """
    best, errors, best_t, its = None, [], 0, []
    target = W_hat
    for t in range(iters + 1):
        sp = svd_split(target, rank)
        ev = split_error(W_hat, sp["L1b"], sp["L2b"], fmt)
        errors.append(ev["err"])
        if keep_iterates:
            its.append(dict(target=target, L1=sp["L1"], L2=sp["L2"], L1b=sp["L1b"], L2b=sp["L2b"], err=ev["err"]))
        if best is None or ev["err"] < best["err"]:
            best = dict(L1=sp["L1"], L2=sp["L2"], L1b=sp["L1b"], L2b=sp["L2b"], **ev)
            best_t = t
        target = W_hat - ev["D"]
    if keep_iterates:
        best["iterates"] = its
    return best, errors, best_t


def pack_codes(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Nibble-pack 4-bit codes along the last axis (INT4 as sign-magnitude nibbles)."""
    if fmt == "int4":
        return quant.pack_nibbles(quant.int4_to_nibble(codes))
    return quant.pack_nibbles(codes)


def pack_weights(W_bits: np.ndarray, act_absmax, alpha: float, rank: int, fmt: str, refine_iters: int = 0):
    """Offline pack of one layer: s, W_hat, SVD split, R quantization.

    act_absmax None means no smoothing (s = 1).  refine_iters > 0 takes the split from
    refine_split (then also: errors, the iterates' E, and best_iter).  Returns a dict with
      s64, s32, inv_s32   smoothing factor (fp64, stored fp32, reciprocal fp32)
      L1b [K][r], L2b [r][N] bf16 values (fp64), and their bit patterns L1_bits, L2_bits
      R (fp64), R32 (fp32) the residual
      codesW [N][K], qW [N][K/2] packed nibbles, sW [K/G][N] (fp16 bits or E8M0)
      sigma   singular values of W_hat; L1, L2 unrounded factors
    """
    K, N = W_bits.shape
    if act_absmax is None:
        s64 = np.ones(K)
        s32 = s64.astype(np.float32)
        inv_s32 = s32.copy()
    else:
        w_absmax = quant.channel_absmax_rows(W_bits)
        s64, s32, inv_s32 = quant.smoothing_factors(act_absmax, w_absmax, alpha)
    W_hat = smoothed_weight(W_bits, s32)
    sp = svd_split(W_hat, rank)
    extra = {}
    if refine_iters > 0:
        best, errors, best_t = refine_split(W_hat, rank, fmt, refine_iters)
        sigma = sp["sigma"]
        sp = dict(L1=best["L1"], L2=best["L2"], L1b=best["L1b"], L2b=best["L2b"], R=best["R"], sigma=sigma)
        extra = dict(errors=errors, best_iter=best_t)
    R32 = sp["R"].astype(np.float32)
    codesW, sW = quantize_residual(R32, fmt)
    if fmt == "nvfp4":
        # level-2 scales: the residual's, and the smoothed calibration activations' (max
        # over channels of fp32(max|X_k| * inv_s_k), fixed offline like s itself)
        extra["S_W"] = residual_tensor_scale(R32)
        # without a calibration statistic (act_absmax None) the activations' level-2
        # scale is 1; callers then set S_X themselves
        extra["S_X"] = (np.float32(1.0) if act_absmax is None else quant.nvfp4_tensor_scale(
            (np.asarray(act_absmax, np.float32) * inv_s32).astype(np.float32).max()))
    return dict(
        fmt=fmt, K=K, N=N, rank=rank, s64=s64, s32=s32, inv_s32=inv_s32, W_hat=W_hat,
        L1=sp["L1"], L2=sp["L2"], L1b=sp["L1b"], L2b=sp["L2b"],
        L1_bits=bf16_value_to_bits(sp["L1b"]), L2_bits=bf16_value_to_bits(sp["L2b"]),
        R=sp["R"], R32=R32, sigma=sp["sigma"],
        codesW=codesW, qW=pack_codes(codesW, fmt), sW=sW, **extra,
    )


def fold_lora(packed: dict, A_bits: np.ndarray, B_bits: np.ndarray, scale: float = 1.0):
    """Concatenate an off-the-shelf LoRA (X A B, acting on unsmoothed X) into the
    low-rank branch, leaving the quantized residual untouched.

    X A B = (X diag(s)^-1)(diag(s) A) B, so the smoothing factor is folded into A:
    L1' = [L1b | bf16(scale * diag(s32) A)], L2' = [L2b ; B].  LoRA scale 1.0 unless
    given (the pages fix none).
    """
    sA = round_f64_to_bf16(float(scale) * np.asarray(packed["s32"], dtype=np.float64)[:, None]
                           * bf16_to_f64(A_bits))
    L1n = np.concatenate([packed["L1b"], sA], axis=1)
    L2n = np.concatenate([packed["L2b"], bf16_to_f64(B_bits)], axis=0)
    out = dict(packed)
    out.update(rank=L1n.shape[1], L1b=L1n, L2b=L2n, L1_bits=bf16_value_to_bits(L1n),
               L2_bits=bf16_value_to_bits(L2n))
    return out
