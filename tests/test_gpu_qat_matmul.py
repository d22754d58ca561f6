"""GPU parity of the coupled-training forward's product, rb_qat_matmul (Y = X What^T), on
each engine: the library's matrix-core kernel, rocBLAS, and the layer's automatic choice.

The reference is the product's definition evaluated in fp64 on the exact operand values (the
fp16/bf16 inputs widened): |Y - ref| <= 2e-5 * S + u_out * |ref|, S = |X| |What|^T the sum of
|terms| (the products are exact in fp32; 2e-5 is the fp32 accumulation budget), u_out the
output type's unit roundoff. Shapes are ragged against the 128 x 256 output tiles and cover
K from one 32-column tile up; the 2048 x 4096 x 11008 training shape is checked on sampled outputs.
"""
import numpy as np
import pytest
import torch

import residual_binarized_weight_amd as rb
import workloads as wl
from tests.gpu_util import dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs the GPU")]

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}
UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
ENGINES = {"mfma": rb.RB_QAT_ENGINE_MFMA, "rocblas": rb.RB_QAT_ENGINE_ROCBLAS, "auto": rb.RB_QAT_ENGINE_AUTO}


def operands(seed: int, M: int, N: int, K: int, dt: str, ldx: int | None = None, ldw: int | None = None):
    """X [M][K] (rows ldx apart) and What [N][K] (rows ldw apart) on the device in `dt`, and
    their exact values in fp64. What holds +-g0 +-g1-like values: sums of two scaled signs."""
    rng = np.random.default_rng(seed)
    x = wl.activations(seed, M, K, dtype=np.float32)
    w = (np.sign(rng.standard_normal((N, K))) * 0.03 + np.sign(rng.standard_normal((N, K))) * 0.011).astype(np.float32)
    w *= rng.uniform(0.5, 2.0, size=(1, K)).astype(np.float32)
    out = []
    for a, ld in ((x, ldx), (w, ldw)):
        rows, cols = a.shape
        full = torch.zeros((rows, ld or cols), dtype=TORCH_DT[dt])
        full[:, :cols] = torch.from_numpy(a).to(TORCH_DT[dt])
        view = full.to(dev())[:, :cols]
        out += [view, view.float().cpu().numpy().astype(np.float64)]
    return out


def check(Y: torch.Tensor, ref: np.ndarray, S: np.ndarray, ydt: str):
    v = Y.float().cpu().numpy().astype(np.float64)
    err = np.abs(v - ref)
    tol = 2e-5 * S + UNIT[ydt] * np.abs(ref) + 1e-30
    worst = np.max(err / tol)
    assert worst <= 1.0, f"error {worst:.3f} x tolerance"


@pytest.mark.parametrize("engine", ["mfma", "rocblas", "auto"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ydt", ["f32", "act"])
@pytest.mark.parametrize("M,N,K", [(1, 96, 64), (130, 300, 1056), (257, 513, 2080), (64, 256, 32)])
def test_matmul_matches_definition(engine, dt, ydt, M, N, K):
    X, Xv, Wh, Whv = operands(600 + M, M, N, K, dt)
    y_dtype = torch.float32 if ydt == "f32" else TORCH_DT[dt]
    Y = rb.qat_matmul(X, Wh, y_dtype=y_dtype, engine=ENGINES[engine])
    torch.cuda.synchronize()
    check(Y, Xv @ Whv.T, np.abs(Xv) @ np.abs(Whv).T, "f32" if ydt == "f32" else dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_matmul_strided_rows_and_output(dt):
    """Operand rows ldx / ldwh apart (ldx > K, ldwh > K, multiples of 8) and an output with
    ldy > N: the columns past N of Y are not written."""
    M, N, K = 200, 270, 768
    X, Xv, Wh, Whv = operands(611, M, N, K, dt, ldx=K + 24, ldw=K + 8)
    Yfull = torch.full((M, N + 5), 7.0, dtype=torch.float32, device=dev())
    Y = Yfull[:, :N]
    rb.qat_matmul(X, Wh, Y=Y, engine=rb.RB_QAT_ENGINE_MFMA)
    torch.cuda.synchronize()
    check(Y, Xv @ Whv.T, np.abs(Xv) @ np.abs(Whv).T, "f32")
    assert torch.all(Yfull[:, N:] == 7.0)


def test_matmul_kernel_rejects_unsupported_layouts():
    """The matrix-core engine needs K to be a multiple of 32 (whole K tiles) and the row strides
    multiples of 8 (whole 16-byte chunks); the automatic engine falls back to rocBLAS."""
    M, N, K = 33, 70, 300
    X, Xv, Wh, Whv = operands(612, M, N, K, "bf16")
    with pytest.raises(rb.RbError):
        rb.qat_matmul(X, Wh, y_dtype=torch.float32, engine=rb.RB_QAT_ENGINE_MFMA)
    Y = rb.qat_matmul(X, Wh, y_dtype=torch.float32, engine=rb.RB_QAT_ENGINE_AUTO)
    torch.cuda.synchronize()
    check(Y, Xv @ Whv.T, np.abs(Xv) @ np.abs(Whv).T, "f32")
    X2, Xv2, Wh2, Whv2 = operands(615, M, N, 1000, "bf16")   # a multiple of 8, not of 32
    with pytest.raises(rb.RbError):
        rb.qat_matmul(X2, Wh2, y_dtype=torch.float32, engine=rb.RB_QAT_ENGINE_MFMA)
    Y2 = rb.qat_matmul(X2, Wh2, y_dtype=torch.float32)
    torch.cuda.synchronize()
    check(Y2, Xv2 @ Whv2.T, np.abs(Xv2) @ np.abs(Whv2).T, "f32")


def test_matmul_training_shape_sampled():
    """The 2048-token batch on the 4096 x 11008 layer (the benchmarked launch): 16 sampled
    batch rows x all 4096 outputs, the first and last row included, bf16 output."""
    M, N, K = 2048, 4096, 11008
    X, _, Wh, _ = operands(613, M, N, K, "bf16")
    Y = rb.qat_matmul(X, Wh, engine=rb.RB_QAT_ENGINE_MFMA)
    torch.cuda.synchronize()
    rows = np.concatenate([[0], np.sort(np.random.default_rng(5).choice(np.arange(1, M - 1), 14, replace=False)),
                           [M - 1]])
    Xv = X[rows].float().cpu().numpy().astype(np.float64)
    Whv = Wh.float().cpu().numpy().astype(np.float64)
    check(Y[rows], Xv @ Whv.T, np.abs(Xv) @ np.abs(Whv).T, "bf16")


def test_matmul_is_deterministic():
    M, N, K = 300, 520, 1600
    X, _, Wh, _ = operands(614, M, N, K, "bf16")
    a = rb.qat_matmul(X, Wh, y_dtype=torch.float32, engine=rb.RB_QAT_ENGINE_MFMA)
    b = rb.qat_matmul(X, Wh, y_dtype=torch.float32, engine=rb.RB_QAT_ENGINE_MFMA)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
