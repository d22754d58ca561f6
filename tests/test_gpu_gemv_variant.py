"""GPU parity of rb_gemv_variant ({0, 1} planes and a per-row offset) against the oracle's
gemv_variant, within 1e-3 * sum|terms| (the product rule), on the nibble-table path (M = 1,
fp16, h = 1, k <= 2) and the direct path (other types, M > 1, a general h)."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import assert_product_close, dev, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def planes_of(seed: int, k: int, N: int, K: int) -> np.ndarray:
    W = wl.heavy_tailed_weights(seed, N, K)
    return O.binarize(W, k)["planes"]


def run(planes, g, h, mu, x, K, zero_one, y_dtype):
    k, N, _ = planes.shape
    pt = to_dev(planes)
    gt = to_dev(g)
    ht = None if h is None else to_dev(h)
    mt = None if mu is None else to_dev(mu)
    y = rb.gemv_variant(pt, gt, ht, to_dev(x), K, mu=mt, zero_one=zero_one, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.mark.parametrize("zero_one", [False, True])
@pytest.mark.parametrize("with_mu", [False, True])
@pytest.mark.parametrize("k,N,K", [(1, 37, 300), (2, 256, 4096), (2, 100, 11008), (1, 64, 16384)])
def test_nibble_path_variants(zero_one, with_mu, k, N, K):
    planes = planes_of(800 + K, k, N, K)
    rng = np.random.default_rng(801)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float16)
    mu = rng.normal(0, 0.002, N).astype(np.float16) if with_mu else None
    x = wl.activations(802, 1, K)                                     # fp16
    y = run(planes, g, None, mu, x, K, zero_one, torch.float16)
    y_ref, sabs = O.gemv_variant(planes, g.astype(np.float64), None, None if mu is None else mu.astype(np.float64),
                                 x.astype(np.float64), K, zero_one)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("zero_one", [False, True])
@pytest.mark.parametrize("M,k,general_h,with_mu", [(1, 3, False, True), (4, 2, True, False), (16, 1, False, True),
                                                   (7, 4, True, False), (2, 2, False, False)])
def test_direct_path_variants(zero_one, M, k, general_h, with_mu):
    N, K = 70, 517
    planes = planes_of(810 + M, k, N, K)
    rng = np.random.default_rng(811 + M)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float32)
    h = wl.random_scales(812, k, K, negative_frac=0.1, dtype=np.float32) if general_h else None
    mu = rng.normal(0, 0.002, N).astype(np.float32) if with_mu else None
    x = wl.activations(813, M, K, dtype=np.float32)
    y = run(planes, g, h, mu, x, K, zero_one, torch.float32)
    y_ref, sabs = O.gemv_variant(planes, g.astype(np.float64), None if h is None else h.astype(np.float64),
                                 None if mu is None else mu.astype(np.float64), x.astype(np.float64), K, zero_one)
    assert_product_close(y, y_ref, sabs, fp16_out=False)


def test_plain_variant_is_rb_gemv_bit_for_bit():
    N, K, k = 256, 4096, 2
    planes = to_dev(planes_of(820, k, N, K))
    g = to_dev(np.random.default_rng(821).uniform(0.005, 0.03, (k, N)).astype(np.float16))
    x = to_dev(wl.activations(822, 1, K))
    y1 = rb.gemv(planes, g, None, x, K)
    y2 = rb.gemv_variant(planes, g, None, x, K)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_offset_requires_unit_h():
    N, K, k = 16, 64, 1
    planes = to_dev(planes_of(830, k, N, K))
    g = to_dev(np.ones((k, N), np.float32))
    with pytest.raises(rb.RbError):
        rb.gemv_variant(planes, g, to_dev(np.ones((k, K), np.float32)), to_dev(np.ones((1, K), np.float32)), K,
                        mu=to_dev(np.zeros(N, np.float32)), y_dtype=torch.float32)


def test_mlp_down_layer_variants_sampled_rows():
    # the 4096 x 11008 layer, k = 2, M = 1, fp16, in the metric's launch configuration; the
    # oracle on 64 sampled rows
    W = wl.weights_for("down")
    N, K = W.shape
    planes, g = rb.pack(torch.from_numpy(W).to(dev()), 2)
    rng = np.random.default_rng(840)
    mu = rng.normal(0, 0.002, N).astype(np.float16)
    x = wl.activations_for("down", 1)
    rows = np.sort(rng.choice(N, 64, replace=False))
    pl = planes.cpu().numpy().view(np.uint32)[:, rows]
    gn = g.float().cpu().numpy().astype(np.float64)[:, rows]
    for zero_one in (False, True):
        for m in (None, mu):
            y = rb.gemv_variant(planes, g, None, to_dev(x), K, mu=None if m is None else to_dev(m),
                                zero_one=zero_one)
            torch.cuda.synchronize()
            y_ref, sabs = O.gemv_variant(pl, gn, None, None if m is None else m.astype(np.float64)[rows],
                                         x.astype(np.float64), K, zero_one)
            assert_product_close(y.float().cpu().numpy()[:, rows], y_ref, sabs)


@pytest.mark.parametrize("zero_one", [False, True])
@pytest.mark.parametrize("N,K,M", [(1, 1, 1), (1, 64, 3), (5, 1, 16), (3, 33, 1)])
def test_variant_degenerate_shapes(zero_one, N, K, M):
    k = 2
    planes = planes_of(850 + K, k, N, K)
    rng = np.random.default_rng(851)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float16)
    mu = rng.normal(0, 0.002, N).astype(np.float16)
    x = wl.activations(852, M, K)                                     # fp16
    y = run(planes, g, None, mu, x, K, zero_one, torch.float16)
    y_ref, sabs = O.gemv_variant(planes, g.astype(np.float64), None, mu.astype(np.float64), x.astype(np.float64),
                                 K, zero_one)
    assert_product_close(y, y_ref, sabs)


@pytest.mark.parametrize("k", [1, 2, 3])
def test_zero_one_with_general_h_fp16_m1(k):
    # {0, 1} bits with per-column scales at M = 1 (fp16): the chained single-plane passes
    N, K = 130, 4096
    planes = planes_of(860 + k, k, N, K)
    rng = np.random.default_rng(861)
    g = rng.uniform(0.005, 0.03, (k, N)).astype(np.float16)
    h = wl.random_scales(862, k, K, negative_frac=0.2, dtype=np.float16)
    x = wl.activations(863, 1, K)
    y = run(planes, g, h, None, x, K, True, torch.float16)
    y_ref, sabs = O.gemv_variant(planes, g.astype(np.float64), h.astype(np.float64), None, x.astype(np.float64), K,
                                 True)
    assert_product_close(y, y_ref, sabs)
