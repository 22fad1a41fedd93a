"""svdq_linear_forward_noalloc against svdq_linear_forward, through the C ABI.

The allocation-free entry point runs the same kernels with its workspace in the
library's fixed device array, so its output must equal the forward's bit for bit.  Two
calls in a row, the second with fewer tokens (the array keeps the first call's contents,
which the second must not depend on), on both formats; and a layer whose workspace
exceeds the array is refused with nothing launched (Y untouched).
"""
import ctypes

import numpy as np
import pytest

from gpu_helpers import assert_finite, forward_sentinel, layer_from_oracle, log, oracle_pack, sentinel_out, to_dev_bf16

from bit_diffusion_model_amd import svdq
from bit_diffusion_model_amd.workloads import random_layer

pytestmark = pytest.mark.gpu


def _noalloc(lay, X, ydtype=svdq.F32):
    """The entry point called directly through ctypes on a sentinel-filled Y."""
    import torch

    M = X.shape[0]
    Y = sentinel_out(M, lay.N, ydtype)
    st = svdq.lib().svdq_linear_forward_noalloc(lay.c_layer(), M, ctypes.c_void_p(X.data_ptr()), X.stride(0),
                                                 ctypes.c_void_p(Y.data_ptr()), Y.stride(0), ydtype,
                                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, svdq.lib().svdq_last_error().decode()
    return Y


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_noalloc_matches_forward_twice(fmt):
    import torch

    K, N, r = 3072, 1536, 32
    wl = random_layer(4608, K, N, r, 99 if fmt == "int4" else 98, fmt=fmt, x_out=31, w_out=0)
    lay = layer_from_oracle(oracle_pack(wl))
    X = to_dev_bf16(wl.X)
    for M in (4608, 777):  # the second call smaller than the first
        for ydt in (svdq.F32, svdq.BF16):
            log(f"noalloc {fmt} M={M} ydtype={ydt}")
            Xm = X[:M]
            Yn = _noalloc(lay, Xm, ydt)
            Yf, _ = forward_sentinel(lay, Xm, ydt)
            torch.cuda.synchronize()
            assert_finite(Yn)
            assert torch.equal(Yn.view(torch.int16 if ydt == svdq.BF16 else torch.int32),
                               Yf.view(torch.int16 if ydt == svdq.BF16 else torch.int32)), "differs from the forward"
    # the same bits when the calls alternate with the forward on another layer
    wl2 = random_layer(300, 256, 200, 8, 5, fmt=fmt, x_out=2)
    lay2 = layer_from_oracle(oracle_pack(wl2))
    X2 = to_dev_bf16(wl2.X)
    a = _noalloc(lay2, X2)
    b = _noalloc(lay, X[:777])
    c = _noalloc(lay2, X2)
    assert torch.equal(a, c) and torch.equal(b, forward_sentinel(lay, X[:777])[0])


def test_noalloc_refuses_beyond_the_array():
    import torch

    K, N = 12288, 8192
    lay = svdq.PackedLinear(K, N, 0, svdq.INT4_G64, np.ones(K, np.float32), np.zeros((0, K), np.uint16),
                            np.zeros((0, N), np.uint16), np.zeros((N, K // 2), np.uint8),
                            np.zeros((K // 64, N), np.uint16))
    M = 8192  # 8192 x 12288 bytes of operand codes alone exceed 64 MiB
    assert svdq.lib().svdq_workspace_bytes(lay.c_layer(), M) > svdq.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda:0")
    st = svdq.lib().svdq_linear_forward_noalloc(lay.c_layer(), M, ctypes.c_void_p(X.data_ptr()), K,
                                                 ctypes.c_void_p(Y.data_ptr()), N, svdq.F32,
                                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 2 and b"scratch" in svdq.lib().svdq_last_error()
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all()), "nothing may be launched"
