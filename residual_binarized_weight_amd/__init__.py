"""Residual binarized weights on AMD Instinct MI355X: Python face of librb.

Thin wrappers over the C ABI in include/rb.h. PyTorch provides device buffers and the
current HIP stream; every computation runs in librb's HIP kernels. Functions take and
return CUDA (HIP) tensors on the current device and enqueue on the current stream.

  planes, g = pack(W, k)                         residual sign planes + row scales
  y = gemv(planes, g, h, x, K)                   y = sum_i g_i (.) (B_i (h_i (.) x)), M <= 16
  y = gemm_small(planes, g, h, x, K)             same on the matrix cores, larger M
  y = gemv_variant(planes, g, h, x, K, mu=, zero_one=)   {0, s} planes / per-row offset
  idx = codebook_encode(sign_plane, K, C, v)     nearest binary codeword per v-block
  y = codebook_gemv(idx, C, v, s, group, x, K)   product on codebook indices
  C, idx, M = codebook_learn(sign_plane, K, C0, v, iters)   binary K-means codebook learning
  planes, g, h = svid_init(W, k)                 function-aware initialization of k paths
  planes, What = qat_derive(W, g, h)             coupled training: paths derived from W
  Y, planes, What = qat_forward(W, g, h, X)      ... and the layer's product Y = X What^T
  dW, dX, dg, dh = qat_backward(dY, X, What, planes, g, h)   straight-through backward
  qat_autotune(X, dY, What, Y, dW, dX)           pick the fastest GEMM kernels for a shape
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (RB_F16, RB_F32, RB_BF16, RB_OP_CODEBOOK_GEMV, RB_OP_GEMM_SMALL, RB_OP_GEMV,
                   RB_OP_QAT_BACKWARD, RB_OP_SVID_INIT, RB_QAT_ENGINE_AUTO, RB_QAT_ENGINE_MFMA,
                   RB_QAT_ENGINE_ROCBLAS, RbError, check, lib)

__all__ = ["pack", "gemv", "gemv_variant", "gemm_small", "codebook_encode", "codebook_gemv", "codebook_mstep",
           "codebook_distinct", "codebook_learn", "svid_init", "qat_derive",
           "qat_forward", "qat_matmul", "qat_backward", "qat_autotune", "workspace",
           "workspace_bytes", "storage_bits_per_weight", "version", "RbError", "lib"]

_DT = {torch.float32: RB_F32, torch.float16: RB_F16, torch.bfloat16: RB_BF16}


def _dt(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    return _DT[t]


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("librb takes device tensors")
    if not t.is_contiguous():
        raise ValueError("librb takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _ptr_rows(t: torch.Tensor | None):
    """A matrix whose rows may be strided (unit stride within a row; the row stride is passed
    to the library as the leading dimension)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("librb takes device tensors")
    if t.dim() < 1 or t.stride(-1) != 1 or any(t.stride(d) < 0 for d in range(t.dim())):
        raise ValueError("librb takes matrices with unit stride along rows")
    if t.dim() == 3 and t.stride(0) != t.shape[1] * t.stride(1):
        raise ValueError("librb takes plane stacks with planes stored back to back")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def version() -> int:
    return lib.rb_version()


def workspace_bytes(op: int, k: int, N: int, K: int, M: int) -> int:
    return int(lib.rb_workspace_bytes(op, k, N, K, M))


def storage_bits_per_weight(N: int, K: int, k: int, scale_dtype=torch.float16, has_h: bool = True) -> float:
    return float(lib.rb_storage_bits_per_weight(N, K, k, _dt(scale_dtype), int(has_h)))


def workspace(op: int, k: int, N: int, K: int, M: int, device=None) -> torch.Tensor | None:
    """A zero-filled workspace for the given operation (None when it needs none)."""
    n = workspace_bytes(op, k, N, K, M)
    if n == 0:
        return None
    return torch.zeros((n + 15) // 16 * 16, dtype=torch.uint8, device=device or "cuda")


def pack(W: torch.Tensor, k: int, h: torch.Tensor | None = None, group: int = 0,
         scale_dtype=torch.float16, ldp: int | None = None, planes: torch.Tensor | None = None,
         d_status: torch.Tensor | None = None):
    """Residual sign planes (int32 storage of the uint32 words, [k][N][ldp]) and scales
    ([k][N] or [k][N][ceil(K/group)]) of W [N][K] (fp32/fp16/bf16)."""
    N, K = W.shape
    Kw = (K + 31) // 32
    ldp = Kw if ldp is None else ldp
    if planes is None:
        planes = torch.zeros((k, N, ldp), dtype=torch.int32, device=W.device)
    shape = (k, N) if group == 0 else (k, N, (K + group - 1) // group)
    g = torch.empty(shape, dtype=scale_dtype, device=W.device)
    check("rb_pack", lib.rb_pack(_ptr(W), _dt(W.dtype), N, K, W.stride(0), k, group, _ptr(h),
                                 _dt(scale_dtype), _ptr(planes), ldp, _ptr(g), _ptr(d_status),
                                 _stream()))
    return planes, g


def _product(fn_name: str, planes, g, h, x, K, y_dtype, ws, y, op):
    k, N, ldp = planes.shape
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=x.device)
    if ws is None:
        ws = workspace(op, k, N, K, M, device=x.device)
    fn = getattr(lib, fn_name)
    check(fn_name, fn(_ptr(planes), ldp, _ptr(g), _ptr(h), _dt(g.dtype), k, N, K, _ptr(x),
                      _dt(x.dtype), M, _ptr(y), _dt(y.dtype), _ptr(ws),
                      0 if ws is None else ws.numel(), _stream()))
    return y


def gemv(planes, g, h, x, K: int, y_dtype=torch.float16, ws=None, y=None):
    """y [M][N] = sum_i g_i (.) (B_i (h_i (.) x)) for x [M][K], M <= 16."""
    return _product("rb_gemv", planes, g, h, x, K, y_dtype, ws, y, RB_OP_GEMV)


def gemv_variant(planes, g, h, x, K: int, mu=None, zero_one: bool = False, y_dtype=torch.float16, ws=None,
                 y=None):
    """rb_gemv with {0, 1} planes (zero_one) and/or a per-row offset mu [N] (scale dtype, h None)."""
    k, N, ldp = planes.shape
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=x.device)
    if ws is None:
        ws = workspace(RB_OP_GEMV, k, N, K, M, device=x.device)
    check("rb_gemv_variant", lib.rb_gemv_variant(_ptr(planes), ldp, _ptr(g), _ptr(h), _ptr(mu), int(zero_one),
                                                 _dt(g.dtype), k, N, K, _ptr(x), _dt(x.dtype), M, _ptr(y),
                                                 _dt(y.dtype), _ptr(ws), 0 if ws is None else ws.numel(),
                                                 _stream()))
    return y


def gemm_small(planes, g, h, x, K: int, y_dtype=torch.float16, ws=None, y=None):
    """Same product on the matrix cores, for larger batches (x fp16)."""
    return _product("rb_gemm_small", planes, g, h, x, K, y_dtype, ws, y, RB_OP_GEMM_SMALL)


def codebook_encode(sign_plane: torch.Tensor, K: int, codebook: torch.Tensor, v: int, table: bool = False,
                    ws: torch.Tensor | None = None):
    """uint16 indices (int16 storage) [N][ceil(K/v)] of the nearest codewords; with table=True
    through the nearest-codeword table of all 2^v patterns (v <= 24; same result)."""
    N, ldp = sign_plane.shape
    nb = (K + v - 1) // v
    idx = torch.empty((N, nb), dtype=torch.int16, device=sign_plane.device)
    if not table:
        check("rb_codebook_encode", lib.rb_codebook_encode(_ptr(sign_plane), ldp, N, K, _ptr(codebook),
                                                           codebook.numel(), v, _ptr(idx), _stream()))
        return idx
    if ws is None:
        ws = torch.empty(max(4, lib.rb_codebook_table_bytes(v)), dtype=torch.uint8, device=sign_plane.device)
    check("rb_codebook_encode_table", lib.rb_codebook_encode_table(_ptr(sign_plane), ldp, N, K, _ptr(codebook),
                                                                   codebook.numel(), v, _ptr(idx), _ptr(ws),
                                                                   ws.numel(), _stream()))
    return idx


def codebook_gemv(idx, codebook, v: int, s, group: int, x, K: int, ws=None, y=None):
    N = idx.shape[0]
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    if ws is None:
        ws = workspace(RB_OP_CODEBOOK_GEMV, 1, N, K, M, device=x.device)
    check("rb_codebook_gemv", lib.rb_codebook_gemv(_ptr(idx), _ptr(codebook), codebook.numel(), v,
                                                   _ptr(s), group, N, K, _ptr(x), M, _ptr(y),
                                                   _ptr(ws), 0 if ws is None else ws.numel(),
                                                   _stream()))
    return y


def _learn_ws(N: int, K: int, c: int, v: int, device, ws):
    if ws is None:
        ws = torch.empty(max(4, lib.rb_codebook_learn_workspace_bytes(N, K, c, v)), dtype=torch.uint8, device=device)
    return ws


def codebook_mstep(sign_plane: torch.Tensor, K: int, idx: torch.Tensor, codebook: torch.Tensor, v: int,
                   counts: bool = True, ws: torch.Tensor | None = None):
    """One M-step of binary K-means, in place on `codebook` ([c] int32 storage of the words);
    returns the member count per codeword ([c] int32 storage) or None."""
    N, ldp = sign_plane.shape
    c = codebook.numel()
    cnt = torch.empty(c, dtype=torch.int32, device=codebook.device) if counts else None
    ws = _learn_ws(N, K, c, v, codebook.device, ws)
    check("rb_codebook_mstep", lib.rb_codebook_mstep(_ptr(sign_plane), ldp, N, K, v, _ptr(idx), _ptr(codebook), c,
                                                     _ptr(cnt), _ptr(ws), ws.numel(), _stream()))
    return cnt


def codebook_distinct(sign_plane: torch.Tensor, K: int, codebook: torch.Tensor, v: int,
                      ws: torch.Tensor | None = None) -> torch.Tensor:
    """Number of distinct v-column blocks (a device int32 tensor); if below the codebook size,
    the codebook (in place) becomes those blocks in ascending order."""
    N, ldp = sign_plane.shape
    c = codebook.numel()
    nd = torch.empty(1, dtype=torch.int32, device=codebook.device)
    ws = _learn_ws(N, K, c, v, codebook.device, ws)
    check("rb_codebook_distinct", lib.rb_codebook_distinct(_ptr(sign_plane), ldp, N, K, v, _ptr(codebook), c,
                                                           _ptr(nd), _ptr(ws), ws.numel(), _stream()))
    return nd


def codebook_learn(sign_plane: torch.Tensor, K: int, codebook: torch.Tensor, v: int, iters: int,
                   idx: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Binary K-means from the initial `codebook` (updated in place): returns (codebook, idx
    [N][ceil(K/v)] uint16 as int16 storage, number of distinct blocks as a device int32)."""
    N, ldp = sign_plane.shape
    c = codebook.numel()
    nb = (K + v - 1) // v
    idx = torch.empty((N, nb), dtype=torch.int16, device=codebook.device) if idx is None else idx
    nd = torch.empty(1, dtype=torch.int32, device=codebook.device)
    ws = _learn_ws(N, K, c, v, codebook.device, ws)
    check("rb_codebook_learn", lib.rb_codebook_learn(_ptr(sign_plane), ldp, N, K, v, _ptr(codebook), c, iters,
                                                     _ptr(idx), _ptr(nd), _ptr(ws), ws.numel(), _stream()))
    return codebook, idx, nd


def svid_init(W: torch.Tensor, k: int, T: int = 20, P: int = 4, s_in: torch.Tensor | None = None,
              s_out: torch.Tensor | None = None, a_in: float = 0.0, a_out: float = 0.0,
              ldp: int | None = None, ws: torch.Tensor | None = None):
    """Function-aware initialization of k residual paths of W [N][K] (fp32, row stride a
    multiple of 4): sign planes [k][N][ldp] (int32 storage of the uint32 words) and fp32 scales
    g [k][N], h [k][K], after T Gauss-Seidel sweeps of residual SVID with P power iterations
    per path update; s_in [K] / s_out [N] (fp32, > 0) are the I/O importance vectors."""
    N, K = W.shape
    Kw = (K + 31) // 32
    ldp = Kw if ldp is None else ldp
    if K % 4 != 0 or not W.is_contiguous():
        # rows of a multiple of 4 floats (16-byte rows), as the entry point requires
        Wp = torch.zeros((N, (K + 3) // 4 * 4), dtype=W.dtype, device=W.device)
        Wp[:, :K] = W
        W = Wp
    planes = torch.zeros((k, N, ldp), dtype=torch.int32, device=W.device)
    g = torch.empty((k, N), dtype=torch.float32, device=W.device)
    h = torch.empty((k, K), dtype=torch.float32, device=W.device)
    if ws is None:
        ws = torch.empty((workspace_bytes(RB_OP_SVID_INIT, k, N, K, 1) + 15) // 16 * 16, dtype=torch.uint8,
                         device=W.device)
    check("rb_svid_init", lib.rb_svid_init(_ptr(W), _dt(W.dtype), N, K, W.stride(0), k, T, P, _ptr(s_in),
                                           _ptr(s_out), a_in, a_out, _ptr(planes), ldp, _ptr(g), _ptr(h),
                                           _ptr(ws), ws.numel(), _stream()))
    return planes, g, h


def qat_derive(W: torch.Tensor, g: torch.Tensor, h: torch.Tensor, a_dtype=torch.bfloat16,
               planes: torch.Tensor | None = None, What: torch.Tensor | None = None):
    """Coupled-training derivation: from the shared fp32 weight W [N][K] (rows may be strided)
    and fp32 scales g [k][N], h [k][K], the k sign planes [k][N][ceil(K/32)] (int32 storage)
    and the effective weight What [N][K] in a_dtype (fp16 or bf16)."""
    N, K = W.shape
    k = g.shape[0]
    planes = torch.zeros((k, N, (K + 31) // 32), dtype=torch.int32, device=W.device) if planes is None else planes
    What = torch.empty((N, K), dtype=a_dtype, device=W.device) if What is None else What
    check("rb_qat_derive", lib.rb_qat_derive(_ptr_rows(W), N, K, W.stride(0), k, _ptr(g), _ptr(h), _ptr_rows(planes),
                                             planes.stride(1), _ptr_rows(What), _dt(What.dtype), What.stride(0),
                                             _stream()))
    return planes, What


def qat_forward(W: torch.Tensor, g: torch.Tensor, h: torch.Tensor, X: torch.Tensor, y_dtype=None,
                planes: torch.Tensor | None = None, What: torch.Tensor | None = None,
                Y: torch.Tensor | None = None):
    """Coupled-training forward: the derivation, then Y [M][N] = X What^T for X [M][K] (fp16 or
    bf16, rows may be strided); y_dtype fp32 or X's type (default). Returns (Y, planes, What)."""
    N, K = W.shape
    M = X.shape[0]
    k = g.shape[0]
    planes = torch.zeros((k, N, (K + 31) // 32), dtype=torch.int32, device=W.device) if planes is None else planes
    What = torch.empty((N, K), dtype=X.dtype, device=W.device) if What is None else What
    Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=W.device) if Y is None else Y
    check("rb_qat_forward", lib.rb_qat_forward(_ptr_rows(W), N, K, W.stride(0), k, _ptr(g), _ptr(h), _ptr_rows(X),
                                               _dt(X.dtype), M, X.stride(0), _ptr_rows(planes), planes.stride(1),
                                               _ptr_rows(What), What.stride(0), _ptr_rows(Y), _dt(Y.dtype), Y.stride(0),
                                               _stream()))
    return Y, planes, What


def qat_matmul(X: torch.Tensor, What: torch.Tensor, Y: torch.Tensor | None = None, y_dtype=None,
               engine: int = RB_QAT_ENGINE_AUTO):
    """The coupled-training forward's product alone: Y [M][N] = X What^T for X [M][K] and What
    [N][K] (fp16 or bf16, rows may be strided), Y fp32 or the operand type (default), on
    `engine` (RB_QAT_ENGINE_AUTO, _MFMA: the library's matrix-core kernel, _ROCBLAS)."""
    M, K = X.shape
    N = What.shape[0]
    Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device) if Y is None else Y
    check("rb_qat_matmul", lib.rb_qat_matmul(_ptr_rows(X), _dt(X.dtype), M, X.stride(0), _ptr_rows(What),
                                             What.stride(0), N, K, _ptr_rows(Y), _dt(Y.dtype), Y.stride(0), engine,
                                             _stream()))
    return Y


def qat_backward(dY: torch.Tensor, X: torch.Tensor, What: torch.Tensor, planes: torch.Tensor, g: torch.Tensor,
                 h: torch.Tensor, dx_dtype=None, ws: torch.Tensor | None = None, dW: torch.Tensor | None = None,
                 dX: torch.Tensor | None = None, dg: torch.Tensor | None = None, dh: torch.Tensor | None = None):
    """Coupled-training backward from dY [M][N]: dW = dY^T X (fp32 [N][K]), dX = dY What
    ([M][K], dx_dtype fp32 or the activation type), dg [k][N] and dh [k][K] (fp32)."""
    M, N = dY.shape
    K = X.shape[1]
    k = g.shape[0]
    dev = dY.device
    dW = torch.empty((N, K), dtype=torch.float32, device=dev) if dW is None else dW
    dX = torch.empty((M, K), dtype=dx_dtype or X.dtype, device=dev) if dX is None else dX
    dg = torch.empty((k, N), dtype=torch.float32, device=dev) if dg is None else dg
    dh = torch.empty((k, K), dtype=torch.float32, device=dev) if dh is None else dh
    if ws is None:
        ws = torch.empty(max(16, workspace_bytes(RB_OP_QAT_BACKWARD, k, N, K, M)), dtype=torch.uint8, device=dev)
    check("rb_qat_backward", lib.rb_qat_backward(_ptr_rows(dY), _dt(dY.dtype), M, dY.stride(0), _ptr_rows(X), X.stride(0),
                                                 _ptr_rows(What), What.stride(0), _ptr_rows(planes), planes.stride(1),
                                                 _ptr(g), _ptr(h), k, N, K, _ptr_rows(dW), dW.stride(0), _ptr_rows(dX),
                                                 _dt(dX.dtype), dX.stride(0), _ptr(dg), _ptr(dh), _ptr(ws),
                                                 ws.numel(), _stream()))
    return dW, dX, dg, dh


def qat_autotune(X: torch.Tensor, dY: torch.Tensor, What: torch.Tensor, Y: torch.Tensor, dW: torch.Tensor,
                 dX: torch.Tensor):
    """Time the GEMM kernels rocBLAS offers for this layer shape on these buffers and keep the
    fastest for later qat_forward / qat_backward calls of the same shape (synchronising; Y, dW
    and dX are overwritten)."""
    M, K = X.shape
    N = What.shape[0]
    check("rb_qat_autotune", lib.rb_qat_autotune(_ptr_rows(X), _ptr_rows(dY), _dt(X.dtype), M, X.stride(0),
                                                 dY.stride(0), _ptr_rows(What), What.stride(0), N, K, _ptr_rows(Y),
                                                 _dt(Y.dtype), Y.stride(0), _ptr_rows(dW), dW.stride(0),
                                                 _ptr_rows(dX), _dt(dX.dtype), dX.stride(0), _stream()))

