"""GPU parity of rb_gemm_small (the matrix-core path) against the CPU oracle:
|y - y_ref| <= 1e-3 * sum|terms| for every checked output. Covers the 28672x8192 layer at
batches 64 and 256 (k = 1, 2) on sampled rows, against the M = 1 GEMV on the same packed
weights, and exhaustively checked small cases: ragged N, 64-column stage tails, batch
tails, all plane counts, fp32 scales, general h, negative scales."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import assert_pack_matches, assert_product_close, dev, planes_np, scales_np, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def gpu_gemm(planes, g, h, x, K, y_dtype=torch.float16, sdt=np.float16):
    k, N, _ = planes.shape
    pd = to_dev(planes)
    gd = to_dev(g.reshape(k, N).astype(sdt))
    hd = None if h is None else to_dev(h.astype(np.float16))
    y = rb.gemm_small(pd, gd, hd, to_dev(x.astype(np.float16)), K, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.fixture(scope="module")
def wide_layer():
    """The 28672x8192 layer packed on the GPU with k = 2 (plane 0 alone is the k = 1 case:
    the first plane and scale do not depend on k)."""
    W = wl.weights_for("wide")
    Wd = torch.from_numpy(W).to(dev())
    planes_d, g_d = rb.pack(Wd, 2)
    del Wd
    torch.cuda.synchronize()
    return planes_d, g_d


def test_pack_wide_layer_sampled_rows(wide_layer):
    """The packing these products use, bit-exact against the oracle on 384 sampled rows of
    the 28672x8192 layer (the first and last row included)."""
    planes_d, g_d = wide_layer
    W = wl.weights_for("wide")
    N, K = W.shape
    rows = np.sort(np.random.default_rng(7).choice(np.arange(1, N - 1), 382, replace=False))
    rows = np.concatenate([[0], rows, [N - 1]])
    assert_pack_matches(W, 2, None, "f16", 0, planes_np(planes_d, K), scales_np(g_d, 2, N), rows=rows)


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("M", [64, 256])
def test_gemm_wide_layer_sampled_rows(wide_layer, k, M):
    planes_d, g_d = wide_layer
    N, K = wl.SHAPES["wide"]
    pk, gk = planes_d[:k].contiguous(), g_d[:k].contiguous()
    x = wl.activations_for("wide", M)
    xd = to_dev(x)
    y = rb.gemm_small(pk, gk, None, xd, K).float().cpu().numpy()
    rows = np.sort(np.random.default_rng(1000 + M + k).choice(N, 384, replace=False))
    rows[-1] = N - 1
    planes = planes_np(pk, K)[:, rows]
    g = scales_np(gk, k, N)[:, rows]
    y_ref, sabs = O.gemv(planes, g, None, x, K)
    assert_product_close(y[:, rows], y_ref, sabs)
    # the M = 1 GEMV on the same weights, for every output row of batch row 0
    y1 = rb.gemv(pk, gk, None, xd[:1].contiguous(), K).float().cpu().numpy()
    assert_product_close(y[:1, rows], y1[:, rows].astype(np.float64), 2 * sabs[:1])
    err = np.abs(y[0].astype(np.float64) - y1[0])
    scale = np.abs(x[0].astype(np.float64)).sum() * np.abs(scales_np(gk, k, N)[:, :, 0]).sum(axis=0)
    assert np.all(err <= 2e-3 * scale + 2 * 2.0 ** -25)


@pytest.mark.parametrize("N", [1, 37, 200])
@pytest.mark.parametrize("K", [64, 192, 640])
@pytest.mark.parametrize("M", [1, 33, 64, 100])
def test_gemm_ragged_fold(N, K, M):
    k = 2
    W = wl.heavy_tailed_weights(80, N, K)
    x = wl.activations(81, M, K)
    res = O.binarize(W, k)
    y = gpu_gemm(res["planes"], res["g"], None, x, K, y_dtype=torch.float32)
    y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("M", [5, 300])
def test_gemm_all_plane_counts(k, M):
    N, K = 300, 1088
    W = wl.heavy_tailed_weights(82 + k, N, K)
    x = wl.activations(83, M, K)
    res = O.binarize(W, k)
    y = gpu_gemm(res["planes"], res["g"], None, x, K)
    y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert_product_close(y, y_ref, sabs)


def test_gemm_negative_fp16_scales():
    # the product is defined for any scales: signed g exercises the sign fold
    N, K, M, k = 260, 512, 70, 3
    W = wl.heavy_tailed_weights(84, N, K)
    planes = O.binarize(W, k)["planes"]
    g = wl.random_scales(12, k, N, lo=0.001, hi=0.05, negative_frac=0.4).astype(np.float64)
    x = wl.activations(85, M, K)
    y = gpu_gemm(planes, g, None, x, K, y_dtype=torch.float32)
    y_ref, sabs = O.gemv(planes, g.reshape(k, N, 1), None, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


@pytest.mark.parametrize("M", [33, 100, 300])
def test_gemm_two_planes_one_operand_scale_extremes(M):
    # k = 2, fp16 scales, more than one batch tile: both planes go through one MFMA operand
    # (+-g_0 +-g_1 rounded once to fp16 after a power-of-two rescaling per row). Rows with
    # signed, subnormal, zero, large (|g_0| + |g_1| above the fp16 maximum), cancelling
    # (g_1 = -g_0) and lopsided scales
    N, K, k = 96, 704, 2
    W = wl.heavy_tailed_weights(94, N, K)
    planes = O.binarize(W, k)["planes"]
    rng = np.random.default_rng(95)
    g = np.empty((k, N))
    g[:, 0::8] = rng.uniform(0.001, 0.05, (k, 12)) * rng.choice([-1.0, 1.0], (k, 12))
    g[:, 1::8] = rng.uniform(1e-7, 5e-6, (k, 12))                       # subnormal fp16
    g[0, 2::8], g[1, 2::8] = 0.0, rng.uniform(0.01, 0.02, 12)
    g[:, 3::8] = 0.0
    g[0, 4::8], g[1, 4::8] = rng.uniform(30000, 60000, 12), -rng.uniform(30000, 60000, 12)
    g[0, 5::8] = rng.uniform(0.01, 0.02, 12)
    g[1, 5::8] = -g[0, 5::8]
    g[0, 6::8], g[1, 6::8] = rng.uniform(0.5, 1.0, 12), rng.uniform(1e-6, 1e-5, 12)
    g[0, 7::8], g[1, 7::8] = -rng.uniform(1e-4, 1e-3, 12), rng.uniform(0.1, 0.2, 12)
    g = g.astype(np.float16).astype(np.float64)
    x = wl.activations(96, M, K)
    y = gpu_gemm(planes, g, None, x, K, y_dtype=torch.float32)
    y_ref, sabs = O.gemv(planes, g.reshape(k, N, 1), None, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


@pytest.mark.parametrize("M", [40, 129])
def test_gemm_fp32_scales(M):
    N, K, k = 333, 832, 2
    W = wl.heavy_tailed_weights(86, N, K)
    res = O.binarize(W, k, scale_fmt="f32")
    x = wl.activations(87, M, K)
    y = gpu_gemm(res["planes"], res["g"], None, x, K, y_dtype=torch.float32, sdt=np.float32)
    y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


@pytest.mark.parametrize("M", [17, 96])
def test_gemm_general_h(M):
    N, K, k = 150, 704, 3
    W = wl.heavy_tailed_weights(88, N, K)
    h = wl.random_scales(13, k, K, negative_frac=0.3, dtype=np.float16)
    res = O.binarize(W, k, h=h)
    x = wl.activations(89, M, K)
    y = gpu_gemm(res["planes"], res["g"], h, x, K, y_dtype=torch.float32)
    y_ref, sabs = O.gemv(res["planes"], res["g"], h, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


def test_gemm_padded_ldp_no_writes_past_y_deterministic():
    N, K, M, k = 130, 256, 65, 2
    W = wl.heavy_tailed_weights(90, N, K)
    res = O.binarize(W, k)
    Kw = K // 32
    pad = np.zeros((k, N, Kw + 6), dtype=np.uint32)
    pad[:, :, :Kw] = res["planes"]
    pad[:, :, Kw:] = 0xA5A5A5A5  # words past K must not be read into the product
    pd = to_dev(pad)
    gd = to_dev(res["g"].reshape(k, N).astype(np.float16))
    x = wl.activations(91, M, K)
    xd = to_dev(x)
    buf = torch.full((M * N + 100,), 777.0, dtype=torch.float16, device=dev())
    y = buf[:M * N].view(M, N)
    rb.gemm_small(pd, gd, None, xd, K, y=y)
    y1 = y.clone()
    rb.gemm_small(pd, gd, None, xd, K, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[M * N:] == 777.0)
    assert torch.equal(y1, y)
    y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert_product_close(y.float().cpu().numpy(), y_ref, sabs)


@pytest.mark.parametrize("N,K", [(37, 2048), (300, 4160), (130, 11008)])
@pytest.mark.parametrize("M", [1, 33, 64, 100, 256])
@pytest.mark.parametrize("k", [1, 2])
def test_gemm_k_split_fold(N, K, M, k):
    # few row tiles: the K chunks of a tile run in separate blocks and meet in the workspace
    W = wl.heavy_tailed_weights(92 + k, N, K)
    x = wl.activations(93, M, K)
    res = O.binarize(W, k)
    y = gpu_gemm(res["planes"], res["g"], None, x, K, y_dtype=torch.float32)
    y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


@pytest.mark.parametrize("mode", ["fp32_scales", "general_h"])
@pytest.mark.parametrize("M", [20, 130])
def test_gemm_k_split_other_modes(mode, M):
    N, K, k = 90, 5120, 2
    W = wl.heavy_tailed_weights(94, N, K)
    x = wl.activations(95, M, K)
    if mode == "fp32_scales":
        res = O.binarize(W, k, scale_fmt="f32")
        y = gpu_gemm(res["planes"], res["g"], None, x, K, y_dtype=torch.float16, sdt=np.float32)
        y_ref, sabs = O.gemv(res["planes"], res["g"], None, x, K)
    else:
        h = wl.random_scales(15, k, K, negative_frac=0.3, dtype=np.float16)
        res = O.binarize(W, k, h=h)
        y = gpu_gemm(res["planes"], res["g"], h, x, K, y_dtype=torch.float16)
        y_ref, sabs = O.gemv(res["planes"], res["g"], h, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("M", [64, 256])
def test_gemm_mlp_down_layer_k_split_sampled_rows(M):
    # the 4096 x 11008 layer (32 row tiles): K split across blocks, deterministic
    W = wl.weights_for("down")
    N, K = W.shape
    planes, g = rb.pack(torch.from_numpy(W).to(dev()), 2)
    x = wl.activations_for("down", M)
    xd = to_dev(x)
    y = rb.gemm_small(planes, g, None, xd, K, y_dtype=torch.float32)
    y2 = rb.gemm_small(planes, g, None, xd, K, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = np.sort(np.random.default_rng(96).choice(N, 96, replace=False))
    pl = planes.cpu().numpy().view(np.uint32)[:, rows]
    gn = g.float().cpu().numpy().astype(np.float64)[:, rows].reshape(2, len(rows), 1)
    y_ref, sabs = O.gemv(pl, gn, None, x, K)
    assert_product_close(y.cpu().numpy()[:, rows], y_ref, sabs, fp16_out=False)
