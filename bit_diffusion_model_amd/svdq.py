"""ctypes binding over libsvdq.so (include/svdq.h).

Argument marshalling only: every step of the layer runs in the library (HIP kernels
on the device, C++ on the host).  torch provides device memory and the current HIP
stream; no torch op touches the data on the hot path.  If the library is missing the
import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

INT4_G64, MXFP4_G32, NVFP4_G16 = 0, 1, 2
ACT_PACKED, ACT_MMA = 0, 1  # svdq_act_form
F32, BF16, BF16_GELU = 0, 1, 2  # svdq_dtype (BF16_GELU: bf16 of GELU(y))
MLP_CHAINED, MLP_SEPARATE = 0, 1  # svdq_mlp_mode
FMT = {"int4": INT4_G64, "mxfp4": MXFP4_G32, "nvfp4": NVFP4_G16}
GROUP = {INT4_G64: 64, MXFP4_G32: 32, NVFP4_G16: 16}
MAX_RANK = 128


class SvdqError(RuntimeError):
    pass


class _Layer(ctypes.Structure):
    _fields_ = [
        ("K", ctypes.c_int64), ("N", ctypes.c_int64), ("rank", ctypes.c_int32), ("fmt", ctypes.c_int32),
        ("inv_s", ctypes.c_void_p), ("L1f", ctypes.c_void_p), ("L2f", ctypes.c_void_p), ("qW", ctypes.c_void_p), ("sW", ctypes.c_void_p),
        ("tscale_w", ctypes.c_float), ("tscale_x", ctypes.c_float),
    ]


_lib = None

EXPORTS = [
    "svdq_last_error", "svdq_act_absmax", "svdq_weight_sizes", "svdq_pack_weights", "svdq_pack_weights_refined",
    "svdq_quantize_weights", "svdq_concat_lora", "svdq_prepare_lowrank_down", "svdq_prepare_lowrank",
    "svdq_prepare_weights",
    "svdq_quantize_act_lora_down", "svdq_gemm_w4a4_lora_up", "svdq_gemm_workspace_bytes", "svdq_workspace_bytes",
    "svdq_linear_forward", "svdq_linear_forward_unfused", "svdq_debug_group_sums", "svdq_linear_forward_noalloc",
    "svdq_mlp_workspace_bytes", "svdq_mlp_forward", "svdq_mlp_chain_gemm", "svdq_mlp_chain_reduce",
    "svdq_w4a16_gemm", "svdq_forward_k1_parts",
]
NOALLOC_SCRATCH_BYTES = 64 << 20


def lib():
    """Load libsvdq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SvdqError(f"{LIB_PATH} is missing: build it with bit_diffusion_model_amd.build.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    sig = {
        "svdq_last_error": (ctypes.c_char_p, []),
        "svdq_act_absmax": (I32, [I64, I64, P, I64, P]),
        "svdq_weight_sizes": (I32, [I64, I64, I32, P, P]),
        "svdq_pack_weights": (I32, [I64, I64, P, P, F, I32, I32, P, P, P, P, P, P, P]),
        "svdq_pack_weights_refined": (I32, [I64, I64, P, P, F, I32, I32, I32, P, P, P, P, P, P, P, P]),
        "svdq_quantize_weights": (I32, [I64, I64, P, I32, P, P]),
        "svdq_concat_lora": (I32, [I64, I64, P, I32, P, P, I32, P, P, F, P, P]),
        "svdq_prepare_lowrank_down": (I32, [I64, I32, P, P]),
        "svdq_prepare_lowrank": (I32, [I64, I32, P, P]),
        "svdq_prepare_weights": (I32, [I64, I64, I32, P, P, P, P]),
        "svdq_quantize_act_lora_down": (I32, [P, I64, P, I64, I32, P, P, P, P]),
        "svdq_gemm_w4a4_lora_up": (I32, [P, I64, I32, P, P, P, P, I64, I32, P, ctypes.c_size_t, P]),
        "svdq_gemm_workspace_bytes": (ctypes.c_size_t, [P, I64, I32]),
        "svdq_workspace_bytes": (ctypes.c_size_t, [P, I64]),
        "svdq_forward_k1_parts": (I32, [P, I64]),
        "svdq_linear_forward": (I32, [P, I64, P, I64, P, I64, I32, P, ctypes.c_size_t, P]),
        "svdq_linear_forward_unfused": (I32, [P, I64, P, I64, P, I64, I32, P, ctypes.c_size_t, P]),
        "svdq_debug_group_sums": (I32, [P, I64, I32, P, I64, I64, I64, I64, P, P]),
        "svdq_linear_forward_noalloc": (I32, [P, I64, P, I64, P, I64, I32, P]),
        "svdq_mlp_workspace_bytes": (ctypes.c_size_t, [P, P, I64, I32]),
        "svdq_mlp_forward": (I32, [P, P, I64, P, I64, P, I64, I32, I32, P, ctypes.c_size_t, P]),
        "svdq_mlp_chain_gemm": (I32, [P, P, I64, P, P, P, P, P, P, P, I64, P]),
        "svdq_mlp_chain_reduce": (I32, [P, P, I64, P, P, P]),
        "svdq_w4a16_gemm": (I32, [I64, I64, I64, P, I64, P, P, P, I64, I32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise SvdqError(f"svdq status {status}: {lib().svdq_last_error().decode()}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ host functions

def act_absmax(X_bits: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    out = np.empty(X.shape[1], np.float32)
    _check(lib().svdq_act_absmax(X.shape[0], X.shape[1], _ptr(X), X.shape[1], _ptr(out)))
    return out


def weight_sizes(K: int, N: int, fmt: int):
    q = ctypes.c_size_t()
    s = ctypes.c_size_t()
    _check(lib().svdq_weight_sizes(K, N, fmt, ctypes.byref(q), ctypes.byref(s)))
    return q.value, s.value


@dataclass
class HostPack:
    """Offline pack artifacts (host numpy arrays)."""
    K: int
    N: int
    rank: int
    fmt: int
    s: np.ndarray       # fp32 [K]
    inv_s: np.ndarray   # fp32 [K]
    L1t: np.ndarray     # bf16 bits [rank][K]
    L2: np.ndarray      # bf16 bits [rank][N]
    qW: np.ndarray      # u8 [N][K/2]
    sW: np.ndarray      # fp16 bits u16, E8M0 u8 or E4M3 u8 [K/G][N]
    R: Optional[np.ndarray] = None
    errors: Optional[np.ndarray] = None  # refined packs: each iterate's split error E
    tscale_w: float = 1.0  # NVFP4: the weights' and activations' fp32 tensor scales
    tscale_x: float = 1.0


_PACK_ARRAYS = ("s", "inv_s", "L1t", "L2", "qW", "sW", "R", "errors")


def save_pack(p: HostPack, path: str) -> None:
    """Write a pack's artifacts (the offline result: smoothing factors, low-rank factors,
    residual codes and scales, and the NVFP4 tensor scales) to one .npz file; load_pack
    reads them back bit for bit.  Plain arrays only (no pickled objects)."""
    arrays = {k: getattr(p, k) for k in _PACK_ARRAYS if getattr(p, k) is not None}
    meta = np.array([p.K, p.N, p.rank, p.fmt], dtype=np.int64)
    tsc = np.array([p.tscale_w, p.tscale_x], dtype=np.float32)
    np.savez(path, meta=meta, tscales=tsc, **arrays)


def load_pack(path: str) -> HostPack:
    """Read a pack written by save_pack (numpy's loader with pickles disallowed)."""
    with np.load(path, allow_pickle=False) as z:
        K, N, rank, fmt = (int(v) for v in z["meta"])
        tw, tx = (float(v) for v in z["tscales"])
        opt = {k: (z[k].copy() if k in z.files else None) for k in ("R", "errors")}
        return HostPack(K, N, rank, fmt, z["s"].copy(), z["inv_s"].copy(), z["L1t"].copy(), z["L2"].copy(),
                        z["qW"].copy(), z["sW"].copy(), opt["R"], opt["errors"], tw, tx)


def pack_weights(W_bits: np.ndarray, act_absmax_: Optional[np.ndarray], alpha: float, rank: int,
                 fmt: int, want_R: bool = False, refine_iters: int = 0) -> HostPack:
    """svdq_pack_weights, or with refine_iters > 0 svdq_pack_weights_refined (the
    iterates' errors in .errors)."""
    W = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W.shape
    s = np.empty(K, np.float32)
    inv = np.empty(K, np.float32)
    L1t = np.zeros((rank, K), np.uint16)
    L2 = np.zeros((rank, N), np.uint16)
    qW = np.empty((N, K // 2), np.uint8)
    sbuf, sW = _scale_buffer(K, N, fmt)
    R = np.empty((K, N), np.float32) if want_R else None
    a = None if act_absmax_ is None else np.ascontiguousarray(act_absmax_, dtype=np.float32)
    errs = None
    if refine_iters > 0:
        errs = np.empty(refine_iters + 1, np.float64)
        _check(lib().svdq_pack_weights_refined(K, N, _ptr(W), _ptr(a), float(alpha), rank, fmt, int(refine_iters),
                                               _ptr(s), _ptr(inv), _ptr(L1t), _ptr(L2), _ptr(qW), _ptr(sbuf), _ptr(R),
                                               _ptr(errs)))
    else:
        _check(lib().svdq_pack_weights(K, N, _ptr(W), _ptr(a), float(alpha), rank, fmt, _ptr(s), _ptr(inv),
                                       _ptr(L1t), _ptr(L2), _ptr(qW), _ptr(sbuf), _ptr(R)))
    tw, tx = _tscales(sbuf, K, N, fmt)
    return HostPack(K, N, rank, fmt, s, inv, L1t, L2, qW, sW, R, errs, tw, tx)


def _scale_buffer(K: int, N: int, fmt: int):
    """The pack's scale buffer (NVFP4: group scales, then the two fp32 tensor scales) and
    its [K/G][N] view of the group scales."""
    G = GROUP.get(fmt, 64)
    if fmt == INT4_G64:
        b = np.empty((K // G, N), np.uint16)
        return b, b
    b = np.empty((K // G) * N + (8 if fmt == NVFP4_G16 else 0), np.uint8)
    return b, b[:(K // G) * N].reshape(K // G, N)


def _tscales(sbuf, K: int, N: int, fmt: int):
    if fmt != NVFP4_G16:
        return 1.0, 1.0
    t = sbuf[(K // 16) * N:].view(np.float32)
    return float(t[0]), float(t[1])


def quantize_weights(R: np.ndarray, fmt: int, with_tscale: bool = False):
    """svdq_quantize_weights: (qW, sW) (and the NVFP4 weight tensor scale if asked)."""
    R = np.ascontiguousarray(R, dtype=np.float32)
    K, N = R.shape
    qW = np.empty((N, K // 2), np.uint8)
    sbuf, sW = _scale_buffer(K, N, fmt)
    _check(lib().svdq_quantize_weights(K, N, _ptr(R), fmt, _ptr(qW), _ptr(sbuf)))
    return (qW, sW, _tscales(sbuf, K, N, fmt)[0]) if with_tscale else (qW, sW)


def concat_lora(p: HostPack, A_bits: np.ndarray, B_bits: np.ndarray, scale: float = 1.0) -> HostPack:
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B_bits, dtype=np.uint16)
    lr = A.shape[1]
    r = p.rank + lr
    L1t = np.empty((r, p.K), np.uint16)
    L2 = np.empty((r, p.N), np.uint16)
    _check(lib().svdq_concat_lora(p.K, p.N, _ptr(p.s), p.rank, _ptr(np.ascontiguousarray(p.L1t)),
                                  _ptr(np.ascontiguousarray(p.L2)), lr, _ptr(A), _ptr(B), float(scale),
                                  _ptr(L1t), _ptr(L2)))
    return HostPack(p.K, p.N, r, p.fmt, p.s, p.inv_s, L1t, L2, p.qW, p.sW, p.R, None, p.tscale_w, p.tscale_x)


def r16(rank: int) -> int:
    """rank rounded up to a multiple of 16 (padded width of lora_act, L1f and L2f)."""
    return (rank + 15) // 16 * 16


def prepare_lowrank_down(L1t: np.ndarray):
    """Device layout of the down projection: L1^T [rank][K] in kernel 1's fragment order
    (R16 * K bf16, flat)."""
    r, K = L1t.shape
    L1f = np.zeros((r16(r) * K,), np.uint16)
    _check(lib().svdq_prepare_lowrank_down(K, r, _ptr(np.ascontiguousarray(L1t, dtype=np.uint16)), _ptr(L1f)))
    return L1f


def prepare_lowrank(L2: np.ndarray):
    """Device layout of the up projection: L2 in kernel 2's fragment order (N rounded
    up to 32 times R16 bf16, flat)."""
    L2 = np.ascontiguousarray(L2, dtype=np.uint16)
    r, N = L2.shape
    L2f = np.zeros(((N + 31) // 32 * 32 * r16(r),), np.uint16)
    _check(lib().svdq_prepare_lowrank(N, r, _ptr(L2), _ptr(L2f)))
    return L2f


def pad4(n: int) -> int:
    return (n + 3) // 4 * 4


def prepare_weights(K: int, N: int, fmt: int, qW: np.ndarray, sW: np.ndarray):
    """Kernel layout of the residual weights: (qW bytes: (N rounded up to 2) * K/2 in
    column pairs; sW bytes: INT4 fp16 [K/64][Np]; MXFP4 E8M0 [K/32][Np]; NVFP4 E4M3
    [K/64][Np][4]; Np = N rounded up to 4)."""
    qW = np.ascontiguousarray(qW, dtype=np.uint8)
    sW = np.ascontiguousarray(sW)
    qo = np.empty(((N + 1) // 2 * 2 * (K // 2),), np.uint8)
    so = np.empty((K // GROUP[fmt]) * pad4(N) * (2 if fmt == INT4_G64 else 1), np.uint8)
    _check(lib().svdq_prepare_weights(K, N, fmt, _ptr(qW), _ptr(sW), _ptr(qo), _ptr(so)))
    return qo, so


# ------------------------------------------------------------------ device side

def _torch():
    import torch

    if not torch.cuda.is_available():
        raise SvdqError("no HIP device visible to torch")
    return torch


def _dptr(t) -> Optional[int]:
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def torch_uint8():
    return _torch().uint8


def _upload(a: np.ndarray, device):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


class PackedLinear:
    """A packed layer resident on the GPU, callable through the library's kernels."""

    def __init__(self, K: int, N: int, rank: int, fmt: int, inv_s: np.ndarray, L1t: np.ndarray,
                 L2: np.ndarray, qW: np.ndarray, sW: np.ndarray, device="cuda:0", tscale_w: float = 1.0,
                 tscale_x: float = 1.0):
        self.K, self.N, self.rank, self.fmt = int(K), int(N), int(rank), int(fmt)
        self.tscale_w, self.tscale_x = float(tscale_w), float(tscale_x)
        self.device = device
        self.inv_s = _upload(np.asarray(inv_s, np.float32), device)
        if rank > 0:
            self.L1f = _upload(prepare_lowrank_down(L1t), device)
            self.L2f = _upload(prepare_lowrank(L2), device)
        else:
            self.L1f = self.L2f = None
        qk, sk = prepare_weights(self.K, self.N, self.fmt, qW, sW)
        self.qW = _upload(qk, device)
        self.sW = _upload(sk, device)
        self._c = _Layer(self.K, self.N, self.rank, self.fmt, _dptr(self.inv_s), _dptr(self.L1f),
                         _dptr(self.L2f), _dptr(self.qW), _dptr(self.sW), self.tscale_w, self.tscale_x)

    @classmethod
    def from_host_pack(cls, p: HostPack, device="cuda:0"):
        return cls(p.K, p.N, p.rank, p.fmt, p.inv_s, p.L1t, p.L2, p.qW, p.sW, device, p.tscale_w, p.tscale_x)

    @property
    def group(self) -> int:
        return GROUP[self.fmt]

    def c_layer(self):
        return ctypes.byref(self._c)

    def alloc_act(self, M: int, form: int = ACT_PACKED):
        """Device buffers for kernel 1's outputs in the given activation form."""
        torch = _torch()
        mma6 = form == ACT_MMA and self.fmt == INT4_G64
        if form == ACT_MMA and not mma6:
            # MXFP4 MMA form: token pairs; the allocation holds the pair of an odd last
            # token (M rounded up to 2 rows), the view has M rows
            buf = torch.empty(((M + 1) // 2 * 2) * (self.K // 2), dtype=torch.uint8, device=self.device)
            qX = buf[:M * (self.K // 2)].view(M, self.K // 2)
        else:
            qX = torch.empty((M, self.K if mma6 else self.K // 2), dtype=torch.uint8, device=self.device)
        if form == ACT_MMA:  # scales with rows padded to 4: INT4 fp16, MXFP4 E8M0, NVFP4 E4M3 bytes
            sX = torch.empty((self.K // self.group) * pad4(M) * (2 if mma6 else 1), dtype=torch.uint8,
                             device=self.device)
        else:
            sdt = torch.int16 if self.fmt == INT4_G64 else torch.uint8
            sX = torch.empty((self.K // self.group, M), dtype=sdt, device=self.device)
        la = None
        if self.rank:
            if form == ACT_MMA:
                # bf16 hi/lo pairs in fragment order, M rounded up to 32 rows
                la = torch.empty(((M + 31) // 32 * 32 * 2 * r16(self.rank),), dtype=torch.int16,
                                 device=self.device)
            else:
                la = torch.empty((M, r16(self.rank)), dtype=torch.float32, device=self.device)
        return qX, sX, la

    def quantize_act(self, X, out=None, form: int = ACT_PACKED):
        """Kernel 1 on bf16 X [M][K] (torch tensor on the device)."""
        M = X.shape[0]
        qX, sX, la = out if out is not None else self.alloc_act(M, form)
        _check(lib().svdq_quantize_act_lora_down(self.c_layer(), M, _dptr(X), X.stride(0), form, _dptr(qX),
                                                 _dptr(sX), _dptr(la), _stream()))
        return qX, sX, la

    def gemm_workspace(self, M: int, form: int = ACT_PACKED):
        """Device scratch for kernel 2's split of its last round (None when unused)."""
        n = lib().svdq_gemm_workspace_bytes(self.c_layer(), M, form)
        return _torch().empty(n, dtype=torch_uint8(), device=self.device) if n else None

    def gemm(self, qX, sX, la, ydtype: int = F32, out=None, form: int = ACT_PACKED, workspace=None):
        """Kernel 2: Y [M][N] from kernel 1's outputs (same activation form)."""
        torch = _torch()
        M = qX.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float32 if ydtype == F32 else torch.bfloat16,
                              device=self.device)
        nws = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().svdq_gemm_w4a4_lora_up(self.c_layer(), M, form, _dptr(qX), _dptr(sX), _dptr(la),
                                            _dptr(out), out.stride(0), ydtype, _dptr(workspace), nws, _stream()))
        return out

    def workspace(self, M: int):
        torch = _torch()
        n = lib().svdq_workspace_bytes(self.c_layer(), M)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def forward_k1_parts(self, M: int) -> int:
        """svdq_forward_k1_parts: the K ranges the forward cuts kernel 1 into (1: one pass)."""
        return int(lib().svdq_forward_k1_parts(self.c_layer(), M))

    def forward(self, X, ydtype: int = F32, out=None, workspace=None, fused: bool = True):
        """The public layer: svdq_linear_forward (kernel 1 then kernel 2), or with
        fused=False svdq_linear_forward_unfused (the low-rank branch as kernels of its own)."""
        torch = _torch()
        M = X.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float32 if ydtype == F32 else torch.bfloat16,
                              device=self.device)
        ws = workspace if workspace is not None else self.workspace(M)
        fn = lib().svdq_linear_forward if fused else lib().svdq_linear_forward_unfused
        _check(fn(self.c_layer(), M, _dptr(X), X.stride(0), _dptr(out), out.stride(0), ydtype, _dptr(ws), ws.numel(),
                  _stream()))
        return out

    def forward_noalloc(self, X, ydtype: int = F32, out=None):
        """svdq_linear_forward_noalloc: the forward with its workspace in the library's fixed
        device array (no workspace argument, nothing allocated by the library)."""
        torch = _torch()
        M = X.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float32 if ydtype == F32 else torch.bfloat16,
                              device=self.device)
        _check(lib().svdq_linear_forward_noalloc(self.c_layer(), M, _dptr(X), X.stride(0), _dptr(out), out.stride(0),
                                                 ydtype, _stream()))
        return out

    def group_sums(self, qX, m0: int, n0: int, mt: int, nt: int, form: int = ACT_PACKED, out=None):
        """Exact INT4 group sums I[g][m][n] for a window (diagnostic); form ACT_MMA runs the
        forward's own kernel 2 on MMA-form codes."""
        torch = _torch()
        if out is None:
            out = torch.empty((self.K // 64, mt, nt), dtype=torch.int32, device=self.device)
        _check(lib().svdq_debug_group_sums(self.c_layer(), qX.shape[0], form, _dptr(qX), m0, n0, mt, nt,
                                           _dptr(out), _stream()))
        return out


class MlpPair:
    """Two packed layers with GELU between them, Y = fc2(bf16(GELU(fc1(X)))), through
    svdq_mlp_forward (chained or separate) and the chained step's two calls."""

    def __init__(self, fc1: PackedLinear, fc2: PackedLinear):
        if fc1.N != fc2.K:
            raise SvdqError("fc1's N must equal fc2's K")
        self.fc1, self.fc2 = fc1, fc2
        self.device = fc1.device

    def workspace(self, M: int, mode: int = MLP_CHAINED):
        n = lib().svdq_mlp_workspace_bytes(self.fc1.c_layer(), self.fc2.c_layer(), M, mode)
        return _torch().empty(max(n, 256), dtype=torch_uint8(), device=self.device)

    def forward(self, X, ydtype: int = F32, out=None, workspace=None, mode: int = MLP_CHAINED):
        torch = _torch()
        M = X.shape[0]
        if out is None:
            out = torch.empty((M, self.fc2.N), dtype=torch.float32 if ydtype == F32 else torch.bfloat16,
                              device=self.device)
        ws = workspace if workspace is not None else self.workspace(M, mode)
        _check(lib().svdq_mlp_forward(self.fc1.c_layer(), self.fc2.c_layer(), M, _dptr(X), X.stride(0), _dptr(out),
                                      out.stride(0), ydtype, mode, _dptr(ws), ws.numel(), _stream()))
        return out

    def chain_gemm(self, qX, sX, la, M: int, hidden: bool = False, out=None):
        """fc1's kernel 2 with fc2's kernel 1 in its epilogue, on fc1's MMA-form activation
        side.  Returns (qX2, sX2, lora_part, G or None)."""
        torch = _torch()
        K2 = self.fc2.K
        if out is None:
            qX2, sX2, _ = self.fc2.alloc_act(M, ACT_MMA)
            part = (torch.empty(((K2 // 128) * M * r16(self.fc2.rank),), dtype=torch.float32, device=self.device)
                    if self.fc2.rank else None)
            G = torch.empty((M, K2), dtype=torch.bfloat16, device=self.device) if hidden else None
        else:
            qX2, sX2, part, G = out
        _check(lib().svdq_mlp_chain_gemm(self.fc1.c_layer(), self.fc2.c_layer(), M, _dptr(qX), _dptr(sX), _dptr(la),
                                         _dptr(qX2), _dptr(sX2), _dptr(part), _dptr(G),
                                         K2 if G is None else G.stride(0), _stream()))
        return qX2, sX2, part, G

    def chain_reduce(self, part, M: int, out=None):
        """fc2's MMA-form lora_act from the chained step's partials (None when rank 0)."""
        if not self.fc2.rank:
            return None
        la2 = out if out is not None else self.fc2.alloc_act(M, ACT_MMA)[2]
        _check(lib().svdq_mlp_chain_reduce(self.fc1.c_layer(), self.fc2.c_layer(), M, _dptr(part), _dptr(la2),
                                           _stream()))
        return la2


class WeightOnlyLinear:
    """The 4-bit weight-only baseline (svdq_w4a16_gemm): W's own INT4 codes and fp16 group
    scales on the GPU, upcast to bf16 inside the kernel."""

    def __init__(self, K: int, N: int, qW: np.ndarray, sW: np.ndarray, device="cuda:0"):
        self.K, self.N, self.device = int(K), int(N), device
        self.qW = _upload(np.asarray(qW, np.uint8), device)
        self.sW = _upload(np.asarray(sW, np.uint16), device)

    @classmethod
    def from_weights(cls, W_bits: np.ndarray, device="cuda:0") -> "WeightOnlyLinear":
        """Quantize W (bf16 bits [K][N]) with the library's INT4 group quantizer
        (svdq_quantize_weights) and upload the codes and scales."""
        W = np.ascontiguousarray(W_bits, dtype=np.uint16)
        Wf = (W.astype(np.uint32) << 16).view(np.float32)
        qW, sW = quantize_weights(Wf, INT4_G64)
        return cls(W.shape[0], W.shape[1], qW, sW, device)

    def forward(self, X, ydtype: int = F32, out=None):
        torch = _torch()
        M = X.shape[0]
        if out is None:
            out = torch.empty((M, self.N), dtype=torch.float32 if ydtype == F32 else torch.bfloat16,
                              device=self.device)
        _check(lib().svdq_w4a16_gemm(M, self.K, self.N, _dptr(X), X.stride(0), _dptr(self.qW), _dptr(self.sW),
                                     _dptr(out), out.stride(0), ydtype, _stream()))
        return out
