"""w12_gemm_noalloc -- w12_gemm whose K-split workspace is the library's fixed per-GPU
scratch array, for callers that cannot allocate -- through the C ABI.

GPU: on two calls in a row (the second with fewer rows, on the same scratch array), on a
K-split shape and a whole-K shape, its output equals w12_gemm's bit for bit (same kernels,
same split) and the oracle's acceptance rule holds; a w12_gemm with its own workspace
between the two changes nothing.  Host: argument errors and a workspace need beyond
W12_NOALLOC_SCRATCH_BYTES are rejected before any HIP call."""
import ctypes

import numpy as np
import pytest

from oracle import w12_oracle as o
import w12_inputs as wi
from gpu_util import say, to_dev, to_host

FAKE = 0x10000          # non-null, aligned, never dereferenced (validation fails first)


def _call(L, x_ptr, m, d, y_ptr, stream=None):
    return L.w12_gemm_noalloc(ctypes.c_void_p(x_ptr), m, ctypes.byref(d), ctypes.c_void_p(y_ptr),
                              stream)


def test_noalloc_rejects_on_host():
    import lossless_bit_weight_w12_amd as w12
    from lossless_bit_weight_w12_amd import w12 as B
    L = w12.lib()

    def desc(n, k):
        d = B.W12Desc()
        d.n, d.k, d.n_esc = n, k, 0
        for i in range(16):
            d.codebook[i] = 100 + i
        d.e_max = 120
        d.tiles = d.esc_off = FAKE
        d.esc = None
        return d
    assert _call(L, 0, 1, desc(1024, 1024), FAKE) == -1               # x NULL
    assert _call(L, FAKE, 1, desc(1024, 1024), 0) == -1               # y NULL
    assert _call(L, FAKE, 0, desc(1024, 1024), FAKE) == -3            # m outside 1..128
    assert _call(L, FAKE, 1, desc(1000, 1024), FAKE) == -2            # n % 16
    assert _call(L, FAKE + 2, 1, desc(1024, 1024), FAKE) == -7        # x misaligned
    # a K-split launch whose workspace exceeds the scratch array: W12_ERR_WORKSPACE
    n, k, m = 16384, 4096, 128
    need = w12.workspace_bytes(w12.OP_GEMM, m, n, k)
    assert need > w12.NOALLOC_SCRATCH_BYTES
    assert _call(L, FAKE, m, desc(n, k), FAKE) == -5
    # the largest decode-size launch of the MLP block fits
    assert w12.workspace_bytes(w12.OP_GEMM, 32, 5120, 17408) <= w12.NOALLOC_SCRATCH_BYTES


@pytest.mark.gpu
@pytest.mark.parametrize("n,k", [(320, 4096), (5120, 17408), (2080, 512)])
def test_noalloc_equals_gemm_two_calls(n, k):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import lossless_bit_weight_w12_amd as w12
    L = w12.lib()
    g = np.random.default_rng(8100 + n)
    w = wi.gaussian_bf16((n, k), 0.02, g)
    t = w12.encode(to_dev(w, torch))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for m in (32, 8):                          # the second call is smaller
        x = wi.gaussian_bf16((m, k), 1.0, g)
        xt = to_dev(x, torch)
        say("noalloc", n, k, m, "workspace", w12.workspace_bytes(w12.OP_GEMM, m, n, k))
        y = torch.full((m, n), -1, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
        d = t.desc()
        assert _call(L, xt.data_ptr(), m, d, y.data_ptr(), stream) == 0
        y_ref = w12.gemm(xt, t)                # w12_gemm with its own workspace
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (n, k, m)
        z, s = o.gemm_reference(x, w)
        assert o.gemm_accept(to_host(y), z, s).all()
