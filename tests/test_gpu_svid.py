"""GPU parity of rb_svid_init (function-aware initialization: I/O-importance scaling and
iterative residual SVID) against the CPU oracle.

Only the products g_i h_i^T are fixed by the fit; both sides split them evenly
(||g|| = ||h||), so g and h are compared directly. The GPU runs fp32 power iteration and
the oracle an fp64 SVD, so a sign can differ where the residual is within rounding of 0;
such flips must be rare and the fits they feed stay close. Checked per case: g and h
within 1e-4 of the largest entry, at most 1e-4 of the bits flipped, every flip at a
residual that the oracle's own final state puts within 1e-4 of the row's scale, and the
objective ||W' - sum_i What_i|| within 1e-4 relative of the oracle's."""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import assert_product_close, dev, planes_np, to_dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]


def gpu_svid(W, k, T, P=8, s_in=None, s_out=None, a_in=0.0, a_out=0.0):
    N, K = W.shape
    planes, g, h = rb.svid_init(torch.from_numpy(W.astype(np.float32)).to(dev()), k, T=T, P=P,
                                s_in=None if s_in is None else to_dev(s_in.astype(np.float32)),
                                s_out=None if s_out is None else to_dev(s_out.astype(np.float32)),
                                a_in=a_in, a_out=a_out)
    torch.cuda.synchronize()
    return planes, planes_np(planes, K), g.cpu().numpy().astype(np.float64), h.cpu().numpy().astype(np.float64)


def objective(W, B, g, h, fo, fi):
    Wp = fo[:, None] * W * fi[None, :]
    rec = sum(B[i] * np.outer(g[i] * fo, h[i] * fi) for i in range(len(g)))
    return float(np.linalg.norm(Wp - rec))


def check_against_oracle(W, k, T, s_in=None, s_out=None, a_in=0.0, a_out=0.0, P=8, gh_tol=1e-4, flip_tol=1e-4,
                         obj_tol=1e-4):
    N, K = W.shape
    ref = O.svid_init(W.astype(np.float64), k, T=T, s_in=s_in, s_out=s_out, a_in=a_in, a_out=a_out)
    _, pl, g, h = gpu_svid(W, k, T, P, s_in, s_out, a_in, a_out)
    B = np.stack([O.unpack_bits(pl[i], K) for i in range(k)])
    fo = np.ones(N) if s_out is None else s_out.astype(np.float32).astype(np.float64) ** a_out
    fi = np.ones(K) if s_in is None else s_in.astype(np.float32).astype(np.float64) ** a_in
    for i in range(k):
        assert np.max(np.abs(g[i] - ref["g"][i])) <= gh_tol * np.max(np.abs(ref["g"][i])), f"g of path {i}"
        assert np.max(np.abs(h[i] - ref["h"][i])) <= gh_tol * np.max(np.abs(ref["h"][i])), f"h of path {i}"
    flips = B != ref["B"]
    assert flips.sum() <= max(2, 1e-4 * B.size), f"{flips.sum()} of {B.size} bits differ"
    if flips.any():
        # a flip is only allowed where the oracle's final residual of that path is near 0
        Wp = fo[:, None] * W.astype(np.float64) * fi[None, :]
        What = ref["B"] * np.einsum("in,ik->ink", ref["gp"], ref["hp"])
        for (i, n, c) in zip(*np.nonzero(flips)):
            R = Wp[n, c] - (What[:, n, c].sum() - What[i, n, c])
            assert abs(R) <= flip_tol * ref["gp"][i, n] * np.max(ref["hp"][i]), f"flip at {(i, n, c)}, R = {R}"
    obj = objective(W.astype(np.float64), B, g, h, fo, fi)
    assert abs(obj - ref["history"][-1]) <= obj_tol * ref["history"][-1]
    return pl, g, h


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("K", [300, 301, 1000])
def test_svid_matches_oracle(k, K):
    W = wl.heavy_tailed_weights(400 + k, 96, K)
    check_against_oracle(W, k, T=3)


@pytest.mark.parametrize("k", [1, 2])
def test_svid_io_scaling_matches_oracle(k):
    rng = np.random.default_rng(410 + k)
    N, K = 130, 517
    W = wl.heavy_tailed_weights(411, N, K)
    s_in, s_out = rng.lognormal(0, 0.7, K), rng.lognormal(0, 0.5, N)
    check_against_oracle(W, k, T=4, s_in=s_in, s_out=s_out, a_in=0.5, a_out=0.3)


def test_svid_recovers_sign_times_rank1_magnitude():
    rng = np.random.default_rng(420)
    a, b = rng.uniform(0.5, 2.0, 70), rng.uniform(0.1, 3.0, 260)
    S = np.where(rng.random((70, 260)) < 0.5, -1.0, 1.0)
    W = (S * np.outer(a, b)).astype(np.float32)
    _, pl, g, h = gpu_svid(W, 1, T=1, P=6)
    assert np.array_equal(O.unpack_bits(pl[0], 260), S)
    assert np.allclose(np.outer(g[0], h[0]), np.outer(a, b), rtol=2e-5, atol=0)


def test_svid_deterministic_zero_rows_and_padding():
    W = wl.heavy_tailed_weights(430, 40, 203)
    W[7] = 0.0
    p1, pl1, g1, h1 = gpu_svid(W, 2, T=2)
    p2, _, g2, h2 = gpu_svid(W, 2, T=2)
    assert torch.equal(p1, p2) and np.array_equal(g1, g2) and np.array_equal(h1, h2)
    # an all-zero row: zero scales, all signs +1; padding bits past K are 0
    assert np.all(g1[:, 7] == 0.0)
    assert np.all(O.unpack_bits(pl1[:, 7], 203) == 1.0)
    words = p1.cpu().numpy().view(np.uint32)
    assert np.all(words[:, :, -1] >> (203 - 32 * (words.shape[2] - 1)) == 0)


def test_svid_then_product():
    # the initialized paths drive the product with a general h: rb_gemv against the oracle's
    # product on the same planes and scales
    W = wl.heavy_tailed_weights(440, 200, 640)
    planes, pl, g, h = gpu_svid(W, 2, T=3)
    x = wl.activations(441, 3, 640)
    y = rb.gemv(planes, to_dev(g.astype(np.float32)), to_dev(h.astype(np.float32)), to_dev(x), 640,
                y_dtype=torch.float32)
    y_ref, sabs = O.gemv(pl, g.reshape(2, 200, 1), h, x, 640)
    assert_product_close(y.float().cpu().numpy(), y_ref, sabs, fp16_out=False)


def test_svid_mlp_down_layer_two_sweeps():
    # the 4096 x 11008 layer at k = 2: two sweeps against the oracle (fp64 ARPACK SVD)
    W = wl.weights_for("down")
    check_against_oracle(W, 2, T=2, P=4)


def test_svid_down_layer_width_twenty_sweeps():
    # the benched setting, T = 20 sweeps of P = 4 power steps, at the 11008-wide rows of the
    # 4096 x 11008 layer (512 of its rows, so the fp64 oracle finishes in seconds).
    # Twenty alternating sweeps amplify rounding: the same iteration run in fp32 with NumPy
    # on this input departs from the fp64 oracle by up to 1.05e-3 (h) and 1.1e-4 (g) of the
    # largest entry and flips 36 bits at residuals up to 6.3e-4 g max h, while its objective
    # agrees to 9e-8 (in fp64, 4 power steps match the exact SVD to 1e-11). The bounds are
    # those figures with about 3x headroom; the objective, which the fit minimises, keeps a
    # tight bound.
    W = wl.weights_for("down", N=512)
    check_against_oracle(W, 2, T=20, P=4, gh_tol=3e-3, flip_tol=2e-3, obj_tol=1e-5)
