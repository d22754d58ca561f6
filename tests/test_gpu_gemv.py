"""GPU parity of rb_gemv (and cross-feeding with rb_pack) against the CPU oracle:
|y - y_ref| <= 1e-3 * sum|terms| for every output."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import assert_product_close, dev, planes_np, scales_np, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def oracle_case(W, k, h=None, fmt="f16"):
    res = O.binarize(W, k, h=h, scale_fmt=fmt)
    return res["planes"], res["g"]


def gpu_gemv(planes, g, h, x, K, y_dtype=torch.float16, fmt="f16", ldp=None):
    k, N, Kw = planes.shape
    if ldp is not None and ldp != Kw:
        pad = np.zeros((k, N, ldp), dtype=np.uint32)
        pad[:, :, :Kw] = planes
        planes = pad
    sdt = np.float16 if fmt == "f16" else np.float32
    pd = to_dev(planes)
    gd = to_dev(g.reshape(k, N).astype(sdt))
    hd = None if h is None else to_dev(h.astype(sdt))
    xd = to_dev(x)
    y = rb.gemv(pd, gd, hd, xd, K, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def test_gemv_tiny_fp32():
    W = wl.weights_for("tiny")
    x = wl.activations_for("tiny", 1)
    planes, g = oracle_case(W, 1, fmt="f32")
    y = gpu_gemv(planes, g, None, x, 512, y_dtype=torch.float32, fmt="f32")
    y_ref, sabs = O.gemv(planes, g, None, x, 512)
    assert_product_close(y, y_ref, sabs, fp16_out=False)
    # config special case: y = alpha (.) (B x)
    B = O.unpack_bits(planes[0], 512)
    assert np.allclose(y_ref[0], g[0, :, 0] * (B @ x[0].astype(np.float64)), rtol=1e-12, atol=1e-12)


def test_gemv_square_m1():
    W = wl.weights_for("square")
    x = wl.activations_for("square", 1)
    planes, g = oracle_case(W, 2)
    y = gpu_gemv(planes, g, None, x, 4096)
    y_ref, sabs = O.gemv(planes, g, None, x, 4096)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("name", ["down", "gateup"])
@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemv_mlp(name, M):
    W = wl.weights_for(name)
    N, K = W.shape
    rows = np.arange(N) if M == 1 else np.random.default_rng(M).choice(N, 1024, replace=False)
    # pack on the GPU (all rows), compare the product against the oracle on the GPU's planes
    Wd = torch.from_numpy(W).to(dev())
    planes_d, g_d = rb.pack(Wd, 2)
    x = wl.activations_for(name, M)
    y = rb.gemv(planes_d, g_d, None, to_dev(x), K).float().cpu().numpy()
    planes = planes_np(planes_d, K)
    g = scales_np(g_d, 2, N)
    y_ref, sabs = O.gemv(planes[:, rows], g[:, rows], None, x, K)
    assert_product_close(y[:, rows], y_ref, sabs)


@pytest.mark.parametrize("K", [1, 31, 33, 1000, 2049, 4099])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("M", [1, 3])
def test_gemv_ragged(K, k, M):
    N = 37
    W = wl.heavy_tailed_weights(70 + k, N, K)
    x = wl.activations(71, M, K)
    planes, g = oracle_case(W, k)
    y = gpu_gemv(planes, g, None, x, K)
    y_ref, sabs = O.gemv(planes, g, None, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_gemv_general_h_fp32_x(fmt):
    K, N, k = 1500, 70, 3
    W = wl.heavy_tailed_weights(72, N, K)
    sdt = np.float16 if fmt == "f16" else np.float32
    h = wl.random_scales(11, k, K, negative_frac=0.3, dtype=sdt)
    x = wl.activations(73, 2, K, dtype=np.float32)
    planes, g = oracle_case(W, k, h=h, fmt=fmt)
    y = gpu_gemv(planes, g, h, x, K, y_dtype=torch.float32, fmt=fmt)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


def test_gemv_single_row_and_padded_ldp():
    K = 700
    W = wl.heavy_tailed_weights(74, 1, K)
    x = wl.activations(75, 1, K)
    planes, g = oracle_case(W, 2)
    y = gpu_gemv(planes, g, None, x, K, ldp=40)
    y_ref, sabs = O.gemv(planes, g, None, x, K)
    assert_product_close(y, y_ref, sabs)


def test_gemv_writes_nothing_past_y_and_is_deterministic():
    W = wl.weights_for("square", N=600, K=1000)
    x = wl.activations(76, 2, 1000)
    planes, g = oracle_case(W, 2)
    pd, gd, xd = to_dev(planes), to_dev(g.reshape(2, 600).astype(np.float16)), to_dev(x)
    buf = torch.full((2 * 600 + 64,), 12345.0, dtype=torch.float16, device=dev())
    y = buf[:1200].view(2, 600)
    rb.gemv(pd, gd, None, xd, 1000, y=y)
    y1 = y.clone()
    rb.gemv(pd, gd, None, xd, 1000, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[1200:] == 12345.0)
    assert torch.equal(y1, y)
    y_ref, sabs = O.gemv(planes, g, None, x, 1000)
    assert_product_close(y.float().cpu().numpy(), y_ref, sabs)


@pytest.mark.parametrize("N,K,k", [(600, 1000, 2), (4113, 4096, 2), (9000, 4096, 1), (5000, 11001, 2)])
def test_gemv_m1_writes_nothing_past_y_and_is_deterministic(N, K, k):
    # the M = 1 table kernels with 1, 2 and 3 rows per wave and 1 or 3 table phases; N not a
    # multiple of the block's rows; repeated calls bit-identical; nothing written past y
    W = wl.heavy_tailed_weights(77 + k, N, K)
    x = wl.activations(78, 1, K)
    pd, gd = rb.pack(torch.from_numpy(W).to(dev()), k)
    xd = to_dev(x)
    ws = rb.workspace(rb.RB_OP_GEMV, k, N, K, 1)
    buf = torch.full((N + 64,), 12345.0, dtype=torch.float16, device=dev())
    y = buf[:N].view(1, N)
    rb.gemv(pd, gd, None, xd, K, ws=ws, y=y)
    y1 = y.clone()
    rb.gemv(pd, gd, None, xd, K, ws=ws, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[N:] == 12345.0)
    assert torch.equal(y1, y)
    y_ref, sabs = O.gemv(planes_np(pd, K), scales_np(gd, k, N), None, x, K)
    assert_product_close(y.float().cpu().numpy(), y_ref, sabs)


@pytest.mark.parametrize("N,K,k", [(37, 4097, 1), (300, 6000, 2), (4113, 8192, 2), (1000, 10240, 2),
                                   (4113, 10240, 1), (1000, 10272, 2), (515, 11264, 2), (70, 11008, 1),
                                   (515, 11264, 1), (515, 11296, 1), (300, 11296, 2), (300, 11008, 2),
                                   (300, 11007, 2)])
def test_gemv_m1_one_table_build(N, K, k):
    # the one-build kernel for 4096 < K: 3, 4 or 5 table groups (the last one partial), one or
    # two rows per wave, no tail, a tail of 1 to 32 whole words, and shapes just past the tail's
    # reach (11296: 33 words; 11007: not whole words; both run the phased kernel); repeated calls
    # bit-identical, nothing written past y, every row (or 640 sampled ones, first and last
    # included) against the oracle
    W = wl.heavy_tailed_weights(90 + k, N, K)
    x = wl.activations(91, 1, K)
    pd, gd = rb.pack(torch.from_numpy(W).to(dev()), k)
    xd = to_dev(x)
    buf = torch.full((N + 64,), 12345.0, dtype=torch.float16, device=dev())
    y = buf[:N].view(1, N)
    rb.gemv(pd, gd, None, xd, K, y=y)
    y1 = y.clone()
    rb.gemv(pd, gd, None, xd, K, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[N:] == 12345.0)
    assert torch.equal(y1, y)
    rows = np.arange(N)
    if N * K > 4_000_000 and N > 640:
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N + K).choice(N, 638, replace=False)]))
    y_ref, sabs = O.gemv(planes_np(pd, K)[:, rows], scales_np(gd, k, N)[:, rows], None, x, K)
    assert_product_close(y.float().cpu().numpy()[:, rows], y_ref, sabs)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("K", [300, 301, 4096, 6000, 10240, 11008, 16384])
def test_gemv_general_h_fp16_m1(k, K):
    # per-column scales h (fp16, some negative), one activation row: for k <= 2 and 4096 < K <=
    # 11264 one launch of the one-build kernel with a table build per plane (3 or 5 table groups,
    # with and without the tail), else the single-plane nibble pass per plane (K a multiple of
    # 4) or the direct kernel (K = 301)
    N = 96
    W = wl.heavy_tailed_weights(74 + k, N, K)
    h = wl.random_scales(12 + k, k, K, negative_frac=0.2, dtype=np.float16)
    x = wl.activations(75, 1, K)
    planes, g = oracle_case(W, k, h=h)
    y = gpu_gemv(planes, g, h, x, K)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs)


def test_gemv_general_h_leaves_the_workspace_zero():
    # the h passes chain their sums through the workspace and must leave it zero for the
    # byte-table kernel, which shares it (k = 3, h = 1 at M = 1 runs that kernel)
    N, K = 200, 4096
    W = wl.heavy_tailed_weights(76, N, K)
    h = wl.random_scales(13, 2, K, dtype=np.float16)
    x = wl.activations(77, 1, K)
    p2, g2 = oracle_case(W, 2, h=h)
    p3, g3 = oracle_case(W, 3)
    ws = rb.workspace(rb.RB_OP_GEMV, 3, N, K, 1, device=dev())
    for _ in range(2):
        y2 = rb.gemv(to_dev(p2), to_dev(g2.reshape(2, N).astype(np.float16)), to_dev(h), to_dev(x), K, ws=ws)
        y3 = rb.gemv(to_dev(p3), to_dev(g3.reshape(3, N).astype(np.float16)), None, to_dev(x), K, ws=ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws) == 0
        r2, s2 = O.gemv(p2, g2, h, x, K)
        r3, s3 = O.gemv(p3, g3, None, x, K)
        assert_product_close(y2.float().cpu().numpy(), r2, s2)
        assert_product_close(y3.float().cpu().numpy(), r3, s3)


@pytest.mark.parametrize("M", [2, 5, 16])
def test_gemv_general_h_fp16_small_batch(M):
    N, K, k = 70, 1024, 2
    W = wl.heavy_tailed_weights(78, N, K)
    h = wl.random_scales(14, k, K, negative_frac=0.2, dtype=np.float16)
    x = wl.activations(79, M, K)
    planes, g = oracle_case(W, k, h=h)
    y = gpu_gemv(planes, g, h, x, K)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("general_h", [False, True])
@pytest.mark.parametrize("M", [2, 3, 4, 7, 16])
def test_gemv_batches_on_both_sides_of_the_matrix_core_switch(M, general_h):
    # fp16, K a multiple of 64, small planes (K <= 4096): M = 2 runs as nibble passes per row,
    # M >= 3 (K >= 2 N) on the matrix cores (K split into chunks that meet in the workspace)
    N, K, k = 300, 2048, 2
    W = wl.heavy_tailed_weights(90 + M, N, K)
    h = wl.random_scales(91, k, K, negative_frac=0.2, dtype=np.float16) if general_h else None
    x = wl.activations(92 + M, M, K)
    planes, g = oracle_case(W, k, h=h)
    y = gpu_gemv(planes, g, h, x, K)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("N,K,k", [(300, 11008, 2), (4113, 8192, 2), (37, 6000, 1), (515, 11264, 1),
                                   (1000, 10240, 2), (200, 10272, 2), (70, 6001, 2)])
def test_gemv_two_rows_one_launch(N, K, k):
    # M = 2, h = 1, 4096 < K: one launch of the one-build kernel that builds and looks up the
    # tables once per activation row (3, 4 or 5 table groups, with and without the tail; K = 6001
    # is not a multiple of 8 and takes another path); nothing written past y, repeated calls
    # bit-identical, every row (or 640 sampled ones) of both outputs against the oracle
    W = wl.heavy_tailed_weights(99 + k, N, K)
    x = wl.activations(100, 2, K)
    pd, gd = rb.pack(torch.from_numpy(W).to(dev()), k)
    xd = to_dev(x)
    ws = rb.workspace(rb.RB_OP_GEMV, k, N, K, 2)
    buf = torch.full((2 * N + 64,), 12345.0, dtype=torch.float16, device=dev())
    y = buf[:2 * N].view(2, N)
    rb.gemv(pd, gd, None, xd, K, ws=ws, y=y)
    y1 = y.clone()
    rb.gemv(pd, gd, None, xd, K, ws=ws, y=y)
    torch.cuda.synchronize()
    assert torch.all(buf[2 * N:] == 12345.0)
    assert torch.equal(y1, y)
    rows = np.arange(N)
    if N * K > 4_000_000 and N > 640:
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N + K).choice(N, 638, replace=False)]))
    y_ref, sabs = O.gemv(planes_np(pd, K)[:, rows], scales_np(gd, k, N)[:, rows], None, x, K)
    assert_product_close(y.float().cpu().numpy()[:, rows], y_ref, sabs)


def test_gemv_two_rows_on_large_planes_sampled():
    # 28672 x 8192, k = 1 (2^27 bits and more): M = 2 already runs on the matrix cores; random
    # planes and scales, the oracle on 256 sampled rows
    N, K, k = 28672, 8192, 1
    rng = np.random.default_rng(95)
    planes = rng.integers(0, 2**32, size=(k, N, K // 32), dtype=np.uint32)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float16)
    x = wl.activations(96, 2, K)
    y = rb.gemv(to_dev(planes), to_dev(g), None, to_dev(x), K).float().cpu().numpy()
    rows = np.sort(rng.choice(N, 256, replace=False))
    y_ref, sabs = O.gemv(planes[:, rows], g[:, rows].astype(np.float64), None, x, K)
    assert_product_close(y[:, rows], y_ref, sabs)


def test_gemv_matrix_core_batches_keep_the_lut_region_zero():
    # a batch on the matrix cores writes its K-chunk partials after the region that the M = 1
    # byte-table kernel (k = 3) and the general-h chain need zero; all three share one workspace
    N, K = 512, 4096
    W = wl.heavy_tailed_weights(97, N, K)
    h = wl.random_scales(98, 2, K, dtype=np.float16)
    x1 = wl.activations(99, 1, K)
    x16 = wl.activations(100, 16, K)
    p2, g2 = oracle_case(W, 2, h=h)
    p3, g3 = oracle_case(W, 3)
    g2d = to_dev(g2.reshape(2, N).astype(np.float16))
    g3d = to_dev(g3.reshape(3, N).astype(np.float16))
    ws = rb.workspace(rb.RB_OP_GEMV, 3, N, K, 1, device=dev())
    lut = (N * 8 + 255) // 256 * 256
    assert ws.numel() > lut                                  # the partials' region is there
    for _ in range(2):
        y16 = rb.gemv(to_dev(p3), g3d, None, to_dev(x16), K, ws=ws)
        y16h = rb.gemv(to_dev(p2), g2d, to_dev(h), to_dev(x16), K, ws=ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:lut]) == 0
        assert torch.count_nonzero(ws[lut:]) > 0            # the K chunks went through it
        y3 = rb.gemv(to_dev(p3), g3d, None, to_dev(x1), K, ws=ws)
        y2 = rb.gemv(to_dev(p2), g2d, to_dev(h), to_dev(x1), K, ws=ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:lut]) == 0
        for y, p, g, hh, x in ((y16, p3, g3, None, x16), (y16h, p2, g2, h, x16), (y3, p3, g3, None, x1),
                               (y2, p2, g2, h, x1)):
            r, s = O.gemv(p, g, hh, x, K)
            assert_product_close(y.float().cpu().numpy(), r, s)


def test_one_workspace_serves_every_call():
    # one buffer of the largest size the calls need, shared by rb_gemm_small (K-chunk
    # partials), rb_svid_init (scratch) and the M = 1 byte-table and general-h products
    # (which need the zero region zero): the scratch users keep out of the zero region
    N, K = 512, 4096
    W = wl.heavy_tailed_weights(101, N, K)
    h = wl.random_scales(102, 2, K, dtype=np.float16)
    x1 = wl.activations(103, 1, K)
    x64 = wl.activations(104, 64, K)
    p2, g2 = oracle_case(W, 2, h=h)
    p3, g3 = oracle_case(W, 3)
    g2d = to_dev(g2.reshape(2, N).astype(np.float16))
    g3d = to_dev(g3.reshape(3, N).astype(np.float16))
    sizes = [rb.workspace_bytes(rb.RB_OP_GEMV, 3, N, K, 1), rb.workspace_bytes(rb.RB_OP_GEMM_SMALL, 3, N, K, 64),
             rb.workspace_bytes(rb.RB_OP_SVID_INIT, 2, N, K, 1)]
    zr = (N * 8 + 255) // 256 * 256
    assert min(sizes) > zr
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=dev())
    Wd = torch.from_numpy(W).to(dev())
    for _ in range(2):
        y64 = rb.gemm_small(to_dev(p3), g3d, None, to_dev(x64), K, ws=ws)
        rb.svid_init(Wd, 2, T=1, P=2, ws=ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:zr]) == 0
        assert torch.count_nonzero(ws[zr:]) > 0
        y3 = rb.gemv(to_dev(p3), g3d, None, to_dev(x1), K, ws=ws)
        y2 = rb.gemv(to_dev(p2), g2d, to_dev(h), to_dev(x1), K, ws=ws)
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws[:zr]) == 0
        for y, p, g, hh, x in ((y64, p3, g3, None, x64), (y3, p3, g3, None, x1), (y2, p2, g2, h, x1)):
            r, sa = O.gemv(p, g, hh, x, K)
            assert_product_close(y.float().cpu().numpy(), r, sa)


@pytest.mark.parametrize("zero_one", [False, True])
@pytest.mark.parametrize("N,K", [(11008, 4096), (5000, 8200), (777, 4100), (33, 12000), (4096, 11008)])
def test_gemv_two_planes_with_h_in_one_pass(N, K, zero_one):
    # k = 2 with fp16 column scales at M = 1: both planes in one nibble pass, plane 1's phases
    # after plane 0's (3, 2 and 1 rows per wave; 1 to 3 phases, ragged N, a short last phase);
    # random planes and scales, the oracle on up to 300 sampled rows
    k = 2
    rng = np.random.default_rng(N + K)
    planes = rng.integers(0, 2**32, size=(k, N, (K + 31) // 32), dtype=np.uint32)
    if K % 32:
        planes[:, :, -1] &= np.uint32((1 << (K % 32)) - 1)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float16)
    h = wl.random_scales(N, k, K, negative_frac=0.2, dtype=np.float16)
    x = wl.activations(K, 1, K)
    y = rb.gemv_variant(to_dev(planes), to_dev(g), to_dev(h), to_dev(x), K, zero_one=zero_one)
    torch.cuda.synchronize()
    rows = np.arange(N) if N <= 300 else np.sort(rng.choice(N, 300, replace=False))
    y_ref, sabs = O.gemv_variant(planes[:, rows], g[:, rows].astype(np.float64), h.astype(np.float64), None,
                                 x.astype(np.float64), K, zero_one)
    assert_product_close(y.float().cpu().numpy()[:, rows], y_ref, sabs)


@pytest.mark.parametrize("fmt,general_h,y_dtype", [("f32", False, torch.float32), ("f32", False, torch.float16),
                                                    ("f16", True, torch.float32), ("f16", False, torch.float32)])
def test_gemv_matrix_core_batches_other_dtypes(fmt, general_h, y_dtype):
    # batches on the matrix cores with fp32 row scales (one accumulator per plane, g applied in
    # fp32), fp16 h, and fp32 outputs
    N, K, k, M = 200, 3072, 2, 8
    W = wl.heavy_tailed_weights(110, N, K)
    h = wl.random_scales(111, k, K, negative_frac=0.2, dtype=np.float16) if general_h else None
    x = wl.activations(112, M, K)
    planes, g = oracle_case(W, k, h=h, fmt=fmt)
    y = gpu_gemv(planes, g, h, x, K, y_dtype=y_dtype, fmt=fmt)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs, fp16_out=y_dtype == torch.float16)


@pytest.mark.parametrize("general_h", [False, True])
@pytest.mark.parametrize("N", [700, 2100])
def test_gemv_three_rows_both_routes(general_h, N):
    # M = 3 on a near-square layer (K < 2 N and N < 2 K) stays on the nibble passes (one per
    # row); with N >= 2 K it runs on the matrix cores
    K, k, M = 1024, 2, 3
    W = wl.heavy_tailed_weights(120, N, K)
    h = wl.random_scales(121, k, K, negative_frac=0.2, dtype=np.float16) if general_h else None
    x = wl.activations(122, M, K)
    planes, g = oracle_case(W, k, h=h)
    y = gpu_gemv(planes, g, h, x, K)
    y_ref, sabs = O.gemv(planes, g, h, x, K)
    assert_product_close(y, y_ref, sabs)
