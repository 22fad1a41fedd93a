"""Shared helpers for the GPU parity tests (imported by test modules, not collected).

Every input to the HIP path comes from the seeded generators and the oracle's own pack
(never the other way round): the oracle pack's s, L1, L2, codes and scales are uploaded
as the layer, and both sides run the forward on the same X.
"""
import sys

import numpy as np

from bit_diffusion_model_amd import svdq
from oracle import forward as oforward, pack as opack, quant as oquant

TOL_Y = 2e-2  # max |Y - Y_ref| <= TOL_Y * RMS(Y_ref)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_pack(wl, rank=None, fold=True):
    a = oquant.channel_absmax_cols(wl.calib)
    p = opack.pack_weights(wl.W, a, wl.alpha, wl.rank if rank is None else rank, wl.fmt)
    if fold and wl.lora_A is not None:
        p = opack.fold_lora(p, wl.lora_A, wl.lora_B)
    return p


def layer_from_oracle(p, device="cuda:0"):
    fmt = svdq.FMT[p["fmt"]]
    L1t = np.ascontiguousarray(p["L1_bits"].T)
    return svdq.PackedLinear(p["K"], p["N"], p["rank"], fmt, p["inv_s32"], L1t, p["L2_bits"], p["qW"],
                             p["sW"], device)


def to_dev_bf16(X_bits, device="cuda:0"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(X_bits).view(np.int16)).to(device).view(torch.bfloat16)


def oracle_k1(X_bits, p):
    """Oracle kernel-1 outputs in the library's storage layout."""
    Xh, codes, sc = oforward.quantize_activations(X_bits, p["inv_s32"], p["fmt"])
    qX = opack.pack_codes(codes, p["fmt"])
    sX = np.ascontiguousarray(sc.T)  # group-major [K/G][M]
    la = oforward.lora_down(Xh, p["L1b"]) if p["rank"] else None
    return Xh, codes, sc, qX, sX, la


def lora_bound(Xh, L1b):
    """Error budget for X_hat L1 on the GPU: the hi/lo bf16 representation of
    diag(inv_s) L1 (relative 2^-16) plus fp32 accumulation over K terms."""
    K = Xh.shape[1]
    mag = np.abs(Xh.astype(np.float64)) @ np.abs(L1b)
    return (2.0 ** -15 + K * 2.0 ** -23) * mag + 1e-30


def rel_err(Y, Yref):
    rms = np.sqrt(np.mean(Yref ** 2))
    return np.abs(Y - Yref).max() / rms
