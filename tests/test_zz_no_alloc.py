"""rb_gemv_noalloc: rb_gemv with the library's fixed device array as its workspace.

Called through the C ABI and compared with rb_gemv (its own workspace) on the same inputs:
the two run the same kernels, so their outputs must be identical. Two calls in a row, the
second on a smaller problem, and a request beyond the fixed array's size."""
import ctypes

import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from residual_binarized_weight_amd import _lib
from oracle import rb_oracle as O
from tests.gpu_util import assert_product_close, dev, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]

_vp = ctypes.c_void_p
L = _lib.lib

SCRATCH_BYTES = 4 << 20


def noalloc(planes, g, h, x, K, y):
    k, N, ldp = planes.shape
    M = x.shape[0]
    st = L.rb_gemv_noalloc(_vp(planes.data_ptr()), ldp, _vp(g.data_ptr()), _vp(h.data_ptr()) if h is not None else None,
                           _lib.RB_F16, k, N, K, _vp(x.data_ptr()), _lib.RB_F16, M, _vp(y.data_ptr()), _lib.RB_F16,
                           _vp(torch.cuda.current_stream().cuda_stream))
    return st


def case(seed, N, K, k, M, with_h):
    W = wl.heavy_tailed_weights(seed, N, K)
    h = wl.random_scales(seed + 1, k, K, dtype=np.float16) if with_h else None
    res = O.binarize(W, k, h=h)
    x = wl.activations(seed + 2, M, K)
    return res["planes"], res["g"], h, x


@pytest.mark.parametrize("first,second", [
    # (seed, N, K, k, M, h): a batch on the matrix cores (K-chunk partials in the array), then
    # M = 1 on the byte-table kernel (per-row accumulators in the zero region), smaller
    ((300, 4096, 11008, 2, 16, False), (310, 600, 4096, 3, 1, False)),
    # the general-h chain (zero region), then a smaller general-h batch
    ((320, 2048, 8192, 2, 1, True), (330, 500, 2048, 2, 4, True)),
])
def test_noalloc_matches_rb_gemv_on_two_calls(first, second):
    for (seed, N, K, k, M, with_h) in (first, second):
        planes, g, h, x = case(seed, N, K, k, M, with_h)
        pd, gd = to_dev(planes), to_dev(g.reshape(k, N).astype(np.float16))
        hd = None if h is None else to_dev(h)
        xd = to_dev(x)
        y_ref = rb.gemv(pd, gd, hd, xd, K)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev())
        assert noalloc(pd, gd, hd, xd, K, y) == _lib.RB_OK
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"differs from rb_gemv on {(N, K, k, M, with_h)}"
        r, sa = O.gemv(planes, g, h, x, K)
        assert_product_close(y.float().cpu().numpy(), r, sa)


def test_noalloc_rejects_problems_beyond_its_array():
    # 600000 rows need a 4.8 MB zero region (8 bytes per row), more than the 4 MB array
    N, K, k, M = 600000, 64, 1, 1
    assert rb.workspace_bytes(rb.RB_OP_GEMV, k, N, K, M) > SCRATCH_BYTES
    ldp = (K + 31) // 32
    planes = torch.zeros((k, N, ldp), dtype=torch.int32, device=dev())
    g = torch.zeros((k, N), dtype=torch.float16, device=dev())
    x = torch.zeros((M, K), dtype=torch.float16, device=dev())
    y = torch.zeros((M, N), dtype=torch.float16, device=dev())
    assert noalloc(planes, g, None, x, K, y) == _lib.RB_ERR_WORKSPACE
    assert torch.count_nonzero(y) == 0
