"""GPU parity of rb_pack against the CPU oracle (bit-exact planes and scales)."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from tests.gpu_util import assert_pack_matches, dev, planes_np, scales_np, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def run_pack(W, k, h=None, fmt="f16", group=0, ldp=None, wdtype=torch.float32):
    N, K = W.shape
    Wd = torch.from_numpy(W).to(dev()).to(wdtype)
    hd = None if h is None else to_dev(h)
    sdt = torch.float16 if fmt == "f16" else torch.float32
    planes, g = rb.pack(Wd, k, h=hd, group=group, scale_dtype=sdt, ldp=ldp)
    torch.cuda.synchronize()
    return planes, planes_np(planes, K), scales_np(g, k, N)


def test_pack_tiny_fp32_scales():
    W = wl.weights_for("tiny")
    _, p, g = run_pack(W, 1, fmt="f32")
    assert_pack_matches(W, 1, None, "f32", 0, p, g)


def test_pack_square_k2():
    W = wl.weights_for("square")
    _, p, g = run_pack(W, 2)
    assert_pack_matches(W, 2, None, "f16", 0, p, g)


@pytest.mark.parametrize("name", ["down", "gateup"])
def test_pack_mlp_k2_sampled_rows(name):
    W = wl.weights_for(name)
    _, p, g = run_pack(W, 2)
    rows = np.random.default_rng(5).choice(W.shape[0], 384, replace=False)
    assert_pack_matches(W, 2, None, "f16", 0, p, g, rows=rows)


@pytest.mark.parametrize("K", [1, 31, 32, 33, 1000, 2049, 4097])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_pack_ragged_shapes(K, k):
    W = wl.heavy_tailed_weights(40 + k, 9, K)
    _, p, g = run_pack(W, k)
    assert_pack_matches(W, k, None, "f16", 0, p, g)


def test_pack_single_row_and_special_values():
    K = 300
    W = wl.heavy_tailed_weights(50, 6, K)
    W[0] = 0.0                                        # all-zero row: g = 0, all bits +1
    W[1, ::3] = -0.0                                  # negative zeros -> +1
    W[2, :40] = np.float32(1e-40)                     # fp32 subnormals
    W[2, 40:80] = np.float32(-1e-40)
    W[3] = np.where(np.arange(K) % 2 == 0, 0.5, -0.5).astype(np.float32)  # |W| == g exactly
    W[4] = W[3] * np.float32(1.5)
    W[4, 7] = 0.25
    for k in (1, 3):
        _, p, g = run_pack(W, k)
        assert_pack_matches(W, k, None, "f16", 0, p, g)
        _, p1, g1 = run_pack(W[5:6], k)
        assert_pack_matches(W[5:6], k, None, "f16", 0, p1, g1)


@pytest.mark.parametrize("K", [16384, 16385, 20001])
def test_pack_register_row_limit(K):
    # rows up to 16384 columns are held in registers by one block; longer rows take the
    # per-plane traversal: both sides of the limit, with and without h
    W = wl.heavy_tailed_weights(70, 5, K)
    _, p, g = run_pack(W, 2)
    assert_pack_matches(W, 2, None, "f16", 0, p, g)
    h = wl.random_scales(14, 2, K, negative_frac=0.2, dtype=np.float16)
    _, p, g = run_pack(W, 2, h=h)
    assert_pack_matches(W, 2, h, "f16", 0, p, g)


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_pack_general_h_with_negatives(fmt):
    K = 777
    W = wl.heavy_tailed_weights(60, 33, K)
    h = wl.random_scales(9, 3, K, negative_frac=0.3, dtype=np.float16 if fmt == "f16" else np.float32)
    _, p, g = run_pack(W, 3, h=h, fmt=fmt)
    assert_pack_matches(W, 3, h, fmt, 0, p, g)


@pytest.mark.parametrize("wdtype", [torch.float16, torch.bfloat16])
def test_pack_half_precision_inputs(wdtype):
    W32 = wl.heavy_tailed_weights(61, 40, 1100)
    Wt = torch.from_numpy(W32).to(wdtype)
    W = Wt.float().numpy()          # the exact values the GPU sees
    N, K = W.shape
    planes, g = rb.pack(Wt.to(dev()), 2)
    assert_pack_matches(W, 2, None, "f16", 0, planes_np(planes, K), scales_np(g, 2, N))


def test_pack_group16_codebook_scales():
    W = wl.weights_for("codebook", N=256)
    _, p, g = run_pack(W, 1, group=16)
    assert_pack_matches(W, 1, None, "f16", 16, p, g)
    W2 = wl.heavy_tailed_weights(62, 7, 1001)      # ragged last group
    for k in (1, 2):
        _, p, g = run_pack(W2, k, group=16)
        assert_pack_matches(W2, k, None, "f16", 16, p, g)
    _, p, g = run_pack(W2, 1, group=64)
    assert_pack_matches(W2, 1, None, "f16", 64, p, g)


def test_pack_padding_words_untouched():
    W = wl.heavy_tailed_weights(63, 10, 100)
    Kw = 4
    ldp = 8
    planes = torch.full((2, 10, ldp), 0x5A5A5A5A, dtype=torch.int32, device=dev())
    Wd = torch.from_numpy(W).to(dev())
    rb.pack(Wd, 2, ldp=ldp, planes=planes)
    pl = planes.cpu().numpy().view(np.uint32)
    assert np.all(pl[:, :, Kw:] == 0x5A5A5A5A)
    assert_pack_matches(W, 2, None, "f16", 0, pl[:, :, :Kw],
                        scales_np(rb.pack(Wd, 2)[1], 2, 10))


def test_pack_reports_non_finite():
    W = wl.heavy_tailed_weights(64, 5, 200)
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    rb.pack(torch.from_numpy(W).to(dev()), 1, d_status=st)
    assert st.item() == 0
    W[3, 17] = np.inf
    rb.pack(torch.from_numpy(W).to(dev()), 1, d_status=st)
    assert st.item() == 1
    st.zero_()
    W[3, 17] = np.nan
    rb.pack(torch.from_numpy(W).to(dev()), 2, group=16, d_status=st)
    assert st.item() == 1


def test_pack_deterministic():
    W = wl.weights_for("square", N=512)
    a_p, _, a_g = run_pack(W, 2)
    b_p, _, b_g = run_pack(W, 2)
    assert torch.equal(a_p, b_p) and np.array_equal(a_g, b_g)
