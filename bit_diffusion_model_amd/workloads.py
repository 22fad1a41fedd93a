"""Seeded synthetic workloads for the SVDQuant W4A4 + low-rank linear layer.

This module is shared by the HIP path (tests, bench) and by the oracle's tests.
It only *generates data*: Gaussian draws, outlier channels scaled up, the GELU
pre-activation of the MLP's second layer, and the rounding of those draws to the
bf16 storage format.  None of the layer's own arithmetic (smoothing, SVD split,
quantization, GEMM) lives here.

Workload shapes follow the FLUX.1 transformer the SVDQuant abstract (chatpaper.ai,
"SVDQuant: Absorbing Outliers by Low-Rank Components for 4-Bit Diffusion Models")
benchmarks: hidden 3072, 4096 image + 512 text tokens, QKV width 3 x 3072, MLP width
4 x 3072.  Activation outliers sit in a few fixed input channels (the channel-fixed
outlier observation in the "Smooth Quant (W8A8)" section of the ch3chohch3.github.io
post "从 Smooth Quant 到 SVD Quant"), which is what the x30 / x50 channels model.
No real FLUX weights or activations are used: these draws stand in for them.

Recipe (every draw in fp64, outliers scaled in fp64, then fp32 RNE, then bf16 RNE):
  seed = 1000 + config index, numpy SeedSequence(seed).spawn(7) gives independent
  streams for [X, W, X-outlier channels, W-outlier columns, extra batch, LoRA A, LoRA B].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "MlpPair",
    "mlp_pair",
    "make_mlp",
    "CONFIG_NAMES",
    "make",
    "random_layer",
    "bf16_bits_from_f64",
    "bf16_bits_to_f32",
]

# Stream indices in SeedSequence(seed).spawn(7)
_S_X, _S_W, _S_XOUT, _S_WOUT, _S_EXTRA, _S_LA, _S_LB = range(7)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round fp64 draws to fp32 (RNE), then fp32 to bf16 (RNE); returns uint16 bit patterns.

    Storage-format rounding for generated data only (the recipe rounds through fp32).
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    # round-to-nearest-even on the 16 dropped bits; inputs here are finite
    lsb = (u >> 16) & 1
    u = u + 0x7FFF + lsb
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """One linear layer's synthetic inputs.

    X: uint16 [M][K] bf16 bits (tokens x input channels), row-major.
    W: uint16 [K][N] bf16 bits (input channels x output channels), row-major.
    calib: uint16 [Mc][K] bf16 bits, the activations used for the smoothing
           statistic max|X_j| (for most configs the layer's own X).
    lora_A / lora_B: optional uint16 [K][lr] / [lr][N] bf16 bits of an adapter.
    """

    name: str
    M: int
    K: int
    N: int
    rank: int
    fmt: str  # "int4" (INT4, group 64, fp16 scales), "mxfp4" (E2M1, group 32, E8M0 scales) or
    #            "nvfp4" (E2M1, group 16, E4M3 scales under an fp32 tensor scale)
    alpha: float
    X: np.ndarray
    W: np.ndarray
    calib: np.ndarray
    lora_A: Optional[np.ndarray] = None
    lora_B: Optional[np.ndarray] = None
    seed: int = 0
    note: str = ""

    @property
    def group(self) -> int:
        return {"int4": 64, "mxfp4": 32, "nvfp4": 16}[self.fmt]

    @property
    def total_rank(self) -> int:
        return self.rank + (0 if self.lora_A is None else self.lora_A.shape[1])

    def ops_4bit(self) -> int:
        """Algorithmic 4-bit MAC work, counted as 2*M*N*K operations."""
        return 2 * self.M * self.N * self.K


CONFIG_NAMES = ["C0", "C1", "C2a", "C2b", "C3", "C4", "C1nv"]


def _streams(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(7)]


def _outlier_acts(rng_x, rng_c, M, K, n_out, factor, chans=None, base=None):
    x = rng_x.standard_normal((M, K)) if base is None else base
    if chans is None:
        chans = np.sort(rng_c.choice(K, n_out, replace=False))
    x[:, chans] *= factor
    return x, chans


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    # exact erf form of GELU, used only to shape the second MLP layer's input data
    from scipy.special import erf

    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def _c0():
    st = _streams(1000)
    M, K, N = 64, 256, 256
    x, _ = _outlier_acts(st[_S_X], st[_S_XOUT], M, K, 4, 50.0)
    w = st[_S_W].standard_normal((K, N))
    wc = np.sort(st[_S_WOUT].choice(N, 4, replace=False))
    w[:, wc] *= 20.0
    X = bf16_bits_from_f64(x)
    return Workload("C0", M, K, N, 8, "int4", 0.5, X, bf16_bits_from_f64(w), X, seed=1000,
                    note="tiny: 4 activation channels x50, 4 weight output columns x20")


def _c1_parts():
    st = _streams(1001)
    M, K, N = 4608, 3072, 9216
    n_out = round(0.01 * K)
    x, chans = _outlier_acts(st[_S_X], st[_S_XOUT], M, K, n_out, 30.0)
    w = st[_S_W].standard_normal((K, N))
    return bf16_bits_from_f64(x), bf16_bits_from_f64(w), chans


def _c1(fmt="int4", name="C1"):
    X, W, _ = _c1_parts()
    return Workload(name, 4608, 3072, 9216, 32, fmt, 0.5, X, W, X, seed=1001,
                    note="FLUX QKV projection; 31 input channels x30")


def _c2a():
    st = _streams(1002)
    M, K, N = 4608, 3072, 12288
    x, _ = _outlier_acts(st[_S_X], st[_S_XOUT], M, K, round(0.01 * K), 30.0)
    w = st[_S_W].standard_normal((K, N))
    X = bf16_bits_from_f64(x)
    return Workload("C2a", M, K, N, 32, "int4", 0.5, X, bf16_bits_from_f64(w), X, seed=1002,
                    note="FLUX MLP fc1; 31 input channels x30")


def _c2b():
    st = _streams(1002)
    M, K, N = 4608, 12288, 3072
    z = st[_S_EXTRA].standard_normal((M, K))
    x = _gelu_erf(z)
    chans = np.sort(st[_S_WOUT].choice(K, round(0.01 * K), replace=False))
    x[:, chans] *= 30.0
    w = st[_S_LA].standard_normal((K, N))
    X = bf16_bits_from_f64(x)
    return Workload("C2b", M, K, N, 32, "int4", 0.5, X, bf16_bits_from_f64(w), X, seed=1002,
                    note="FLUX MLP fc2; input GELU(N(0,1)), 123 input channels x30")


def _c4():
    X1, W, chans = _c1_parts()
    st = _streams(1004)
    M1, K, N = 4608, 3072, 9216
    x2, _ = _outlier_acts(st[_S_X], None, M1, K, 0, 30.0, chans=chans)
    X2 = bf16_bits_from_f64(x2)
    A = bf16_bits_from_f64(0.02 * st[_S_LA].standard_normal((K, 16)))
    B = bf16_bits_from_f64(0.02 * st[_S_LB].standard_normal((16, N)))
    X = np.concatenate([X1, X2], axis=0)
    # calibration stays on the first batch: the residual branch is not re-quantized
    return Workload("C4", 2 * M1, K, N, 32, "int4", 0.5, X, W, X1, lora_A=A, lora_B=B,
                    seed=1004, note="C1 at batch 2 plus a rank-16 LoRA folded into the low-rank branch")


def make(name: str) -> Workload:
    """Build one of the named workloads (deterministic)."""
    if name == "C0":
        return _c0()
    if name == "C1":
        return _c1()
    if name == "C2a":
        return _c2a()
    if name == "C2b":
        return _c2b()
    if name == "C3":
        return _c1(fmt="mxfp4", name="C3")
    if name == "C4":
        return _c4()
    if name == "C1nv":  # the QKV layer in the group-16 two-level-scale format
        return _c1(fmt="nvfp4", name="C1nv")
    raise KeyError(name)


def random_layer(M: int, K: int, N: int, rank: int, seed: int, fmt: str = "int4",
                 x_out: int = 2, x_factor: float = 30.0, w_out: int = 0, w_factor: float = 20.0,
                 lora_rank: int = 0, alpha: float = 0.5) -> Workload:
    """A small layer with the same value structure as the named configs, any shape."""
    st = _streams(seed)
    x = st[_S_X].standard_normal((M, K))
    if x_out:
        ch = st[_S_XOUT].choice(K, min(x_out, K), replace=False)
        x[:, ch] *= x_factor
    w = st[_S_W].standard_normal((K, N))
    if w_out:
        wc = st[_S_WOUT].choice(N, min(w_out, N), replace=False)
        w[:, wc] *= w_factor
    X = bf16_bits_from_f64(x)
    A = B = None
    if lora_rank:
        A = bf16_bits_from_f64(0.02 * st[_S_LA].standard_normal((K, lora_rank)))
        B = bf16_bits_from_f64(0.02 * st[_S_LB].standard_normal((lora_rank, N)))
    return Workload(f"rand{M}x{K}x{N}r{rank}", M, K, N, rank, fmt, alpha, X,
                    bf16_bits_from_f64(w), X, lora_A=A, lora_B=B, seed=seed)


@dataclasses.dataclass
class MlpPair:
    """Data of a chained MLP pair fc1 -> GELU -> fc2.

    fc1: the first layer's Workload (X is the pair's input).
    fc2: the second layer's weights; its X and calib hold the calibration activations
         for fc2's smoothing (GELU of the unquantized first layer on the first tokens:
         the pair's actual fc2 input is computed by the layers themselves).
    """

    name: str
    fc1: Workload
    fc2: Workload

    @property
    def M(self) -> int:
        return self.fc1.M


def mlp_pair(M: int, K1: int, N1: int, N2: int, r1: int, r2: int, seed: int, x_out: Optional[int] = None,
             h_out: Optional[int] = None, factor: float = 30.0, calib_rows: int = 512, name: str = "") -> MlpPair:
    """A pair with the value structure of the FLUX MLP: fc1's input with x_out outlier
    channels (x factor), fc1's weights N(0,1) scaled so that the hidden pre-activation H
    is about N(0,1) per token (the scale is 1 / sqrt of the mean over tokens of sum_k x_k^2),
    with h_out output columns x factor, so that fc2's input GELU(H) has that many outlier
    channels; fc2's weights N(0,1).  Every draw fp64, rounded through fp32 to bf16."""
    st = _streams(seed)
    n_x = round(0.01 * K1) if x_out is None else x_out
    n_h = round(0.01 * N1) if h_out is None else h_out
    x, _ = _outlier_acts(st[_S_X], st[_S_XOUT], M, K1, n_x, factor)
    X = bf16_bits_from_f64(x)
    xv = bf16_bits_to_f32(X).astype(np.float64)
    w1 = st[_S_W].standard_normal((K1, N1)) / math.sqrt(float(np.mean(np.sum(xv * xv, axis=1))))
    if n_h:
        hc = np.sort(st[_S_WOUT].choice(N1, n_h, replace=False))
        w1[:, hc] *= factor
    W1 = bf16_bits_from_f64(w1)
    w2 = st[_S_LA].standard_normal((N1, N2))
    Mc = min(calib_rows, M)
    h = xv[:Mc] @ bf16_bits_to_f32(W1).astype(np.float64)
    G = bf16_bits_from_f64(_gelu_erf(h))
    fc1 = Workload(f"{name}fc1", M, K1, N1, r1, "int4", 0.5, X, W1, X, seed=seed,
                   note="MLP fc1 of a chained pair")
    fc2 = Workload(f"{name}fc2", Mc, N1, N2, r2, "int4", 0.5, G, bf16_bits_from_f64(w2), G, seed=seed,
                   note="MLP fc2 of a chained pair; X / calib = GELU of the unquantized fc1 on the first tokens")
    return MlpPair(name, fc1, fc2)


def make_mlp(name: str) -> MlpPair:
    """C2chain: the FLUX.1 MLP pair, 4608 tokens, 3072 -> 12288 -> 3072, rank 32 both,
    31 input channels and 123 hidden channels x30 (as the independent fc1 / fc2 layers)."""
    if name == "C2chain":
        return mlp_pair(4608, 3072, 12288, 3072, 32, 32, seed=1005, name="C2chain ")
    raise KeyError(name)
