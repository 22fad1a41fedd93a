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
                             p["sW"], device, float(p.get("S_W", 1.0)), float(p.get("S_X", 1.0)))


def to_dev_bf16(X_bits, device="cuda:0"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(X_bits).view(np.int16)).to(device).view(torch.bfloat16)


def oracle_k1(X_bits, p):
    """Oracle kernel-1 outputs in the library's storage layout."""
    Xh, codes, sc = oforward.quantize_activations(X_bits, p["inv_s32"], p["fmt"], p.get("S_X"))
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


def bf16_rne_bits(v32):
    """fp32 array -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _fp6_fields(words6):
    """[..., 6] uint32 words -> [..., 32] 6-bit fields (field f at bit 6 f)."""
    w = words6.astype(np.uint64)
    out = np.empty(words6.shape[:-1] + (32,), np.int64)
    for f in range(32):
        b, o = divmod(6 * f, 32)
        v = w[..., b] >> np.uint64(o)
        if o > 26:
            v = v | (w[..., b + 1] << np.uint64(32 - o))
        out[..., f] = (v & np.uint64(63)).astype(np.int64)
    return out


def decode_lora_mma(la, M, rank):
    """MMA-form lora_act (device tensor of any integer dtype) -> (hi, lo) bf16 bits [M][R16]
    of the written rows: element ((((m / 32) S + j / 16) 2 + p) 64 + m % 32 + 32 ((j / 8) %
    2)) 8 + j % 8, S = R16 / 16, p = 0 hi, 1 lo."""
    R16 = (rank + 15) // 16 * 16
    M32 = (M + 31) // 32 * 32
    l = la.cpu().numpy().view(np.uint16).reshape(-1)[:M32 * 2 * R16]
    # [m / 32][j / 16][p][j / 8 % 2][m % 32][j % 8] -> [p][m][j]
    l = l.reshape(M32 // 32, R16 // 16, 2, 2, 32, 8).transpose(2, 0, 4, 1, 3, 5).reshape(2, M32, R16)
    return l[0, :M], l[1, :M]


def decode_mma(qX, sX, la, fmt, K, rank, M=None):
    """Kernel 1's MMA-form outputs (device tensors) decoded per the header's description:
    INT4: per token and group 64 bytes, half h at byte 32 h as words [f0 f1 f2 f3 f4 f5 0
    0]; the 192-bit f0..f5 hold 6-bit E2M3 fields (sign bit 5, exponent 0, |q| in bits
    0-2), field f carrying k = 32 h + 16 (f & 1) + (f >> 1); fp16 scale bits [K/64][Mp].
    MXFP4: codes in token pairs (byte b of token m at (m / 2) K + (b / 64) 128 + (m % 2)
    64 + b % 64, M rounded up to 2 rows) and E8M0 bytes [K/32][Mp].  lora_act bf16 hi/lo
    pairs in fragment order: element ((((m / 32) S + j / 16) 2 + p) 64 + m % 32 + 32 ((j /
    8) % 2)) 8 + j % 8, S = R16 / 16, p = 0 hi, 1 lo.  Returns (codes or packed bytes [M][K/2], scales (float64
    values [K/64][M] for INT4, bytes [K/32][M] for MXFP4), hi bits, lo bits)."""
    q = qX.cpu().numpy()
    if M is None:
        M = q.shape[0]
    if fmt != "int4":  # token pairs reach past the M-row view when M is odd
        import torch

        full = torch.empty(0, dtype=torch.uint8, device=qX.device).set_(qX.untyped_storage())
        q = full[qX.storage_offset():].cpu().numpy()
    Mp = (M + 3) // 4 * 4
    sb = None if sX is None else sX.cpu().numpy().view(np.uint8).reshape(-1)
    if fmt == "int4":
        G = K // 64
        w = np.ascontiguousarray(q).view("<u4").reshape(M, G, 2, 8)
        assert not w[..., 6].any() and not w[..., 7].any(), "padding words must be zero"
        fl = _fp6_fields(w[..., :6])
        assert not (fl & 0b011000).any(), "nonzero E2M3 exponent bits"
        v = (fl & 7) * np.where(fl & 32, -1, 1)
        kk = np.array([16 * (f & 1) + (f >> 1) for f in range(32)])
        codes = np.empty_like(v)
        codes[..., kk] = v
        sv = None if sX is None else sb[:G * Mp * 2].view(np.float16).reshape(G, Mp)[:, :M].astype(np.float64)
        out = codes.reshape(M, K), sv
    else:
        M2 = (M + 1) // 2 * 2
        pr = np.ascontiguousarray(q).reshape(-1)[:M2 * K // 2].reshape(M2 // 2, K // 128, 2, 64)
        rows = pr.transpose(0, 2, 1, 3).reshape(M2, K // 2)[:M]
        if fmt == "nvfp4":
            # inside each 64-block code k sits at nibble 2 (16 ((k / 8) % 2) + 4 (k / 16)) + k % 8;
            # scales [K/64][Mp][4]
            nib = np.empty((M, K // 64, 64), np.uint8)
            blk = rows.reshape(M, K // 64, 32)
            for k in range(64):
                pos = 2 * (16 * ((k >> 3) & 1) + 4 * (k >> 4)) + (k & 7)
                nib[:, :, k] = (blk[:, :, pos >> 1] >> (4 * (pos & 1))) & 15
            nib = nib.reshape(M, K)
            rows = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
            sv = None if sX is None else sb[:(K // 64) * Mp * 4].reshape(K // 64, Mp, 4)[:, :M].transpose(0, 2, 1)
            out = rows, (None if sv is None else sv.reshape(K // 16, M))
        else:
            out = rows, sb[:(K // 32) * Mp].reshape(K // 32, Mp)[:, :M]
    hi = lo = None
    if rank:
        hi, lo = decode_lora_mma(la, M, rank)
    return out[0], out[1], hi, lo


# ---------------------------------------------------------------- sentinel buffers
# Every buffer a kernel is meant to write is filled with 0xFF bytes first (NaN for fp32,
# bf16 and fp16; code bytes no kernel writes), so an element a kernel never wrote cannot
# pass as a correct value left over from an earlier allocation.

def sentinel_fill(t):
    """Fill a device tensor's whole allocation (its base, for views) with 0xFF bytes."""
    import torch

    b = t._base if getattr(t, "_base", None) is not None else t
    b.view(torch.uint8).fill_(0xFF) if b.dtype != torch.uint8 else b.fill_(0xFF)
    return t


def sentinel_out(M, N, ydtype=svdq.F32, device="cuda:0"):
    import torch

    Y = torch.empty((M, N), dtype=torch.float32 if ydtype == svdq.F32 else torch.bfloat16, device=device)
    return sentinel_fill(Y)


def sentinel_act(lay, M, form):
    bufs = lay.alloc_act(M, form)
    for t in bufs:
        if t is not None:
            sentinel_fill(t)
    return bufs


def sentinel_ws(lay, M):
    return sentinel_fill(lay.workspace(M))


def sentinel_gemm_ws(lay, M, form):
    w = lay.gemm_workspace(M, form)
    return None if w is None else sentinel_fill(w)


def forward_sentinel(lay, X, ydtype=svdq.F32, fused=True):
    """svdq_linear_forward (or the unfused baseline) with Y and the workspace pre-filled
    with the sentinel; returns (Y, workspace)."""
    M = X.shape[0]
    Y = sentinel_out(M, lay.N, ydtype, X.device)
    ws = sentinel_ws(lay, M)
    lay.forward(X, ydtype, out=Y, workspace=ws, fused=fused)
    return Y, ws


def assert_finite(Y):
    import torch

    bad = int((~torch.isfinite(Y.float())).sum())
    assert bad == 0, f"{bad} outputs not written (sentinel left) or not finite"


# ---------------------------------------------------------------- unit / one-hot scales

F16_ONE = 0x3C00


def unit_scale_layer(p, device="cuda:0"):
    """The oracle pack's residual codes at rank 0 with every weight scale 1.0: kernel 2 then
    returns sum_g sX[m, g] I_g[m, n] exactly, and with activation scales 1.0 or 0.0 an
    exact integer combination of the group sums."""
    K, N = p["K"], p["N"]
    sW = np.full((K // 64, N), F16_ONE, np.uint16)
    return svdq.PackedLinear(K, N, 0, svdq.INT4_G64, p["inv_s32"], np.zeros((0, K), np.uint16),
                             np.zeros((0, N), np.uint16), p["qW"], sW, device)


def mma_scales_int4(M, K, groups_on, device="cuda:0"):
    """MMA-form INT4 activation scales [K/64][Mp] fp16 bits: 1.0 for the groups listed
    (every row), 0.0 elsewhere (padding rows 0)."""
    import torch

    Mp = (M + 3) // 4 * 4
    s = np.zeros((K // 64, Mp), np.uint16)
    for g in groups_on:
        s[g, :M] = F16_ONE
    return torch.from_numpy(s.view(np.uint8).reshape(-1).copy()).to(device)
