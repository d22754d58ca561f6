"""GPU parity of the coupled-training layer (rb_qat_derive / rb_qat_forward / rb_qat_backward)
against the CPU oracle's qat_forward / qat_backward.

Comparison rules:
* planes: bit-exact (both sides take the sign decisions on the fp64 residual in the same
  order);
* What: the GPU value is a nearest fp16/bf16 neighbour of the oracle's fp64 What (error at
  most half a unit in the last place of What's binade; an exact tie must land on the even
  neighbour);
* products (Y, dX): |v - ref| <= (u_a + 2e-5) * S + u_out * |ref|, S the sum of |terms| of
  the oracle's fp64 product, u_a = 2^-p the unit roundoff of the activation type (What's
  rounding), 2e-5 the fp32 accumulation budget, u_out the output's unit roundoff;
* dW: |dW - ref| <= 2e-5 * (|dY|^T |X|) (exact inputs, fp32 accumulation);
* dg, dh: the dW budget carried through the sums, plus 1e-5 of the sum of |terms|.
Inputs X and dY are rounded to the activation type first; the oracle sees those values.
"""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from oracle import rb_oracle as O
from tests.gpu_util import dev, planes_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}
SIG_BITS = {"bf16": 8, "f16": 11}          # significand bits, hidden bit included
MIN_SPACING = {"bf16": 2.0 ** -133, "f16": 2.0 ** -24}
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}   # unit roundoff 2^-p


def act(a32: np.ndarray, dt: str) -> tuple[torch.Tensor, np.ndarray]:
    """The activation tensor on the device in `dt`, and its exact values as fp64."""
    t = torch.from_numpy(np.ascontiguousarray(a32)).to(TORCH_DT[dt])
    return t.to(dev()), t.float().numpy().astype(np.float64)


def assert_nearest(v_dev: torch.Tensor, ref: np.ndarray, dt: str):
    v = v_dev.float().cpu().numpy().astype(np.float64)
    _, e = np.frexp(np.abs(ref))                       # |ref| in [2^(e-1), 2^e)
    spacing = np.maximum(np.ldexp(1.0, e - SIG_BITS[dt]), MIN_SPACING[dt])
    err = np.abs(v - ref)
    bad = err > spacing / 2
    assert not bad.any(), f"{bad.sum()} values not nearest, e.g. {v[bad][:4]} vs {ref[bad][:4]}"
    tie = err == spacing / 2
    if tie.any():
        bits = v_dev.cpu().view(torch.int16).numpy()[tie]
        assert np.all((bits & 1) == 0), "a tie went to the odd neighbour"
    assert np.all(v[ref == 0.0] == 0.0)


def assert_close(v: np.ndarray, ref: np.ndarray, S: np.ndarray, rel: float, u_out: float, what: str):
    err = np.abs(v - ref)
    tol = rel * S + u_out * np.abs(ref) + 1e-30
    worst = np.max(err / tol)
    assert worst <= 1.0, f"{what}: error {worst:.3f} x tolerance"


def layer(seed: int, N: int, K: int, k: int):
    W = wl.heavy_tailed_weights(seed, N, K)
    g, h = wl.training_scales(seed, k, N, K)
    return W, g, h


def derive(W, g, h, dt):
    planes, What = rb.qat_derive(torch.from_numpy(W).to(dev()), torch.from_numpy(g).to(dev()),
                                 torch.from_numpy(h).to(dev()), a_dtype=TORCH_DT[dt])
    torch.cuda.synchronize()
    return planes, What


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("k", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(96, 300), (97, 1000), (40, 301), (8, 64)])
def test_derive_matches_oracle(dt, k, N, K):
    W, g, h = layer(500 + k, N, K, k)
    planes, What = derive(W, g, h, dt)
    _, What_ref, _, planes_ref = O.qat_forward(W, g, h, np.zeros((1, K)))
    assert np.array_equal(planes_np(planes, K), planes_ref)
    assert_nearest(What, What_ref, dt)


def test_derive_sign_of_zero_residuals():
    # W built so that W - g_1 B_1 h_1 is exactly 0 (|W| = g h, both short fp32 values) and W = +-0:
    # every such residual takes sign +1 on both sides
    rng = np.random.default_rng(530)
    N, K, k = 64, 200, 3
    g = (rng.integers(1, 64, size=(k, N)) / 256.0).astype(np.float32)
    h = (rng.integers(1, 64, size=(k, K)) / 64.0).astype(np.float32)
    W = (np.outer(g[0], h[0]) * np.where(rng.random((N, K)) < 0.5, -1.0, 1.0)).astype(np.float32)
    W[::7, ::5] = 0.0
    W[3::7, 2::5] = -0.0
    W[rng.random((N, K)) < 0.2] *= np.float32(1.5)       # and some with a nonzero residual
    planes, What = derive(W, g, h, "bf16")
    _, What_ref, B, planes_ref = O.qat_forward(W, g, h, np.zeros((1, K)))
    assert np.array_equal(planes_np(planes, K), planes_ref)
    assert (B[1] > 0).sum() > N * K // 2                  # the zero residuals took +1
    assert_nearest(What, What_ref, "bf16")


def test_derive_strided_rows_and_padding():
    W, g, h = layer(540, 33, 290, 2)
    Wp = np.zeros((33, 300), np.float32)
    Wp[:, :290] = W
    Wd = torch.from_numpy(Wp).to(dev())[:, :290]
    planes = torch.full((2, 33, 12), -1, dtype=torch.int32, device=dev())
    What_full = torch.full((33, 296), 7, dtype=torch.bfloat16, device=dev())
    What = What_full[:, :290]
    rb.qat_derive(Wd, torch.from_numpy(g).to(dev()), torch.from_numpy(h).to(dev()), planes=planes, What=What)
    torch.cuda.synchronize()
    _, What_ref, _, planes_ref = O.qat_forward(W, g, h, np.zeros((1, 290)))
    pl = planes.cpu().numpy().view(np.uint32)
    assert np.array_equal(pl[..., :10], planes_ref)
    assert np.all(pl[..., 10:] == 0xFFFFFFFF)             # words past ceil(K/32) untouched
    assert_nearest(What, What_ref, "bf16")
    assert torch.all(What_full[:, 290:].float() == 7)      # columns past K untouched


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ydt", ["f32", "act"])
@pytest.mark.parametrize("M,N,K,k", [(1, 96, 300, 2), (7, 130, 1024, 1), (64, 257, 640, 3), (130, 300, 1000, 2)])
def test_forward_matches_oracle(dt, ydt, M, N, K, k):
    W, g, h = layer(550 + M, N, K, k)
    X, Xv = act(wl.activations(550, M, K, dtype=np.float32), dt)
    y_dtype = torch.float32 if ydt == "f32" else TORCH_DT[dt]
    Y, planes, What = rb.qat_forward(torch.from_numpy(W).to(dev()), torch.from_numpy(g).to(dev()),
                                     torch.from_numpy(h).to(dev()), X, y_dtype=y_dtype)
    torch.cuda.synchronize()
    Y_ref, What_ref, _, planes_ref = O.qat_forward(W, g, h, Xv)
    assert np.array_equal(planes_np(planes, K), planes_ref)
    assert_nearest(What, What_ref, dt)
    S = np.abs(Xv) @ np.abs(What_ref).T
    assert_close(Y.float().cpu().numpy(), Y_ref, S, UNIT[dt] + 2e-5, UNIT["f32" if ydt == "f32" else dt], "Y")


def check_backward(W, g, h, Xv, X, dYv, dY, dt, dx_dtype, rows=None, cols=None, y_dtype=torch.float32):
    """Run forward + backward on the GPU and compare with the oracle. rows / cols restrict the
    oracle's work to sampled output rows (dW rows, dg) and input columns (dh, dX columns); the
    derivation is elementwise, so the oracle on a slice of W gives that slice exactly."""
    N, K = W.shape
    k = g.shape[0]
    Wd, gd, hd = (torch.from_numpy(a).to(dev()) for a in (W, g, h))
    _, planes, What = rb.qat_forward(Wd, gd, hd, X, y_dtype=y_dtype)
    dW, dX, dg, dh = rb.qat_backward(dY, X, What, planes, gd, hd, dx_dtype=dx_dtype)
    torch.cuda.synchronize()
    rows = np.arange(N) if rows is None else rows
    cols = np.arange(K) if cols is None else cols
    A = np.abs(dYv).T  # [N][M]
    # dW rows and dg over all columns, for the sampled rows
    _, What_r, B_r, _ = O.qat_forward(W[rows], g[:, rows], h, np.zeros((1, K)))
    dW_r, _, dg_r, _ = O.qat_backward(dYv[:, rows], Xv, What_r, B_r, g[:, rows], h)
    bound_r = 2e-5 * (A[rows] @ np.abs(Xv))
    err = np.abs(dW.cpu().numpy()[rows] - dW_r)
    assert np.all(err <= bound_r + 1e-30), f"dW: {np.max(err / (bound_r + 1e-30)):.3f} x tolerance"
    for i in range(k):
        tol = bound_r @ np.abs(h[i]) + 1e-5 * (np.abs(dW_r) @ np.abs(h[i])) + 1e-30
        e = np.abs(dg.cpu().numpy()[i, rows] - dg_r[i])
        assert np.all(e <= tol), f"dg[{i}]: {np.max(e / tol):.3f} x tolerance"
    # dh and dX for the sampled columns, over all rows
    _, What_c, B_c, _ = O.qat_forward(W[:, cols], g, h[:, cols], np.zeros((1, len(cols))))
    dW_c, dX_c, _, dh_c = O.qat_backward(dYv, Xv[:, cols], What_c, B_c, g, h[:, cols])
    bound_c = 2e-5 * (A @ np.abs(Xv[:, cols]))
    for i in range(k):
        tol = np.abs(g[i]) @ bound_c + 1e-5 * (np.abs(g[i]) @ np.abs(dW_c)) + 1e-30
        e = np.abs(dh.cpu().numpy()[i, cols] - dh_c[i])
        assert np.all(e <= tol), f"dh[{i}]: {np.max(e / tol):.3f} x tolerance"
    dt_out = "f32" if dx_dtype == torch.float32 else dt
    S = np.abs(dYv) @ np.abs(What_c)
    assert_close(dX.float().cpu().numpy()[:, cols], dX_c, S, UNIT[dt] + 2e-5, UNIT[dt_out], "dX")
    return dW, dX, dg, dh


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K,k", [(1, 96, 300, 2), (16, 257, 1000, 2), (33, 130, 517, 4), (64, 300, 777, 1)])
def test_backward_matches_oracle(dt, M, N, K, k):
    W, g, h = layer(560 + k, N, K, k)
    X, Xv = act(wl.activations(560, M, K, dtype=np.float32), dt)
    dY, dYv = act(wl.output_grads(560, M, N), dt)
    check_backward(W, g, h, Xv, X, dYv, dY, dt, torch.float32)
    check_backward(W, g, h, Xv, X, dYv, dY, dt, TORCH_DT[dt])


def test_autotuned_kernels_keep_parity():
    # after choosing the fastest GEMM kernels for a shape, forward and backward still match
    M, N, K, k = 16, 257, 1000, 2
    W, g, h = layer(565, N, K, k)
    X, Xv = act(wl.activations(565, M, K, dtype=np.float32), "bf16")
    dY, dYv = act(wl.output_grads(565, M, N), "bf16")
    What = torch.zeros((N, K), dtype=torch.bfloat16, device=dev())
    rb.qat_autotune(X, dY, What, torch.empty((M, N), dtype=torch.float32, device=dev()),
                    torch.empty((N, K), dtype=torch.float32, device=dev()),
                    torch.empty((M, K), dtype=torch.bfloat16, device=dev()))
    check_backward(W, g, h, Xv, X, dYv, dY, "bf16", torch.bfloat16)


def test_backward_is_deterministic():
    W, g, h = layer(570, 300, 900, 2)
    X, Xv = act(wl.activations(570, 32, 900, dtype=np.float32), "bf16")
    dY, dYv = act(wl.output_grads(570, 32, 300), "bf16")
    Wd, gd, hd = (torch.from_numpy(a).to(dev()) for a in (W, g, h))
    _, planes, What = rb.qat_forward(Wd, gd, hd, X)
    r1 = rb.qat_backward(dY, X, What, planes, gd, hd)
    r2 = rb.qat_backward(dY, X, What, planes, gd, hd)
    torch.cuda.synchronize()
    # dg / dh are fixed-order sums of dW: identical whenever dW is
    if torch.equal(r1[0], r2[0]):
        assert torch.equal(r1[2], r2[2]) and torch.equal(r1[3], r2[3])


def test_mlp_down_layer_training_step_sampled():
    # the 4096 x 11008 layer at k = 2 with 2048 tokens (bf16 activations), as the step is timed:
    # planes and What on sampled rows, Y on sampled tokens and rows, dW / dg on sampled rows,
    # dh / dX on sampled columns
    N, K, k, M = 4096, 11008, 2, 2048
    W = wl.weights_for("down")
    g, h = wl.training_scales(wl.CFG_MLP, k, N, K)
    X, Xv = act(wl.activations(wl.CFG_MLP, M, K, dtype=np.float32), "bf16")
    dY, dYv = act(wl.output_grads(wl.CFG_MLP, M, N), "bf16")
    rs = np.random.default_rng(580)
    rows = np.sort(rs.choice(N, 48, replace=False))
    cols = np.sort(np.concatenate([rs.choice(K - 64, 40, replace=False), np.arange(K - 24, K)]))
    toks = np.sort(rs.choice(M, 6, replace=False))
    Wd, gd, hd = (torch.from_numpy(a).to(dev()) for a in (W, g, h))
    # the kernels the timed step uses: chosen on this shape first
    Y, planes, What = rb.qat_forward(Wd, gd, hd, X)
    rb.qat_autotune(X, dY, What, Y, torch.empty((N, K), dtype=torch.float32, device=dev()),
                    torch.empty((M, K), dtype=torch.bfloat16, device=dev()))
    Y, planes, What = rb.qat_forward(Wd, gd, hd, X)
    torch.cuda.synchronize()
    Y_r, What_r, _, planes_r = O.qat_forward(W[rows], g[:, rows], h, Xv[toks])
    assert np.array_equal(planes_np(planes, K)[:, rows], planes_r)
    assert_nearest(What[torch.from_numpy(rows).to(dev())], What_r, "bf16")
    S = np.abs(Xv[toks]) @ np.abs(What_r).T
    assert_close(Y.float().cpu().numpy()[np.ix_(toks, rows)], Y_r, S, UNIT["bf16"] + 2e-5, UNIT["bf16"], "Y")
    check_backward(W, g, h, Xv, X, dYv, dY, "bf16", torch.bfloat16, rows=rows, cols=cols, y_dtype=torch.bfloat16)


@pytest.mark.parametrize("M,N,K,k", [(1, 1, 1, 1), (1, 1, 33, 4), (3, 5, 1, 2), (2, 7, 64, 3)])
def test_degenerate_shapes(M, N, K, k):
    # one row, one column, one token, and the largest k: every kernel's tail handling
    W, g, h = layer(590 + K, N, K, k)
    X, Xv = act(wl.activations(590, M, K, dtype=np.float32), "bf16")
    dY, dYv = act(wl.output_grads(590, M, N), "bf16")
    Wd, gd, hd = (torch.from_numpy(a).to(dev()) for a in (W, g, h))
    Y, planes, What = rb.qat_forward(Wd, gd, hd, X, y_dtype=torch.float32)
    torch.cuda.synchronize()
    Y_ref, What_ref, _, planes_ref = O.qat_forward(W, g, h, Xv)
    assert np.array_equal(planes_np(planes, K), planes_ref)
    assert_nearest(What, What_ref, "bf16")
    assert_close(Y.cpu().numpy(), Y_ref, np.abs(Xv) @ np.abs(What_ref).T, UNIT["bf16"] + 2e-5, UNIT["f32"], "Y")
    check_backward(W, g, h, Xv, X, dYv, dY, "bf16", torch.float32)
