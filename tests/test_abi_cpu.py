"""The C-ABI library loads and exports every symbol include/rb.h declares, and rejects
invalid calls with the documented status before touching the device (no GPU needed:
validation runs before any HIP call, so these calls never reach a kernel)."""
import ctypes
import os
import re

import pytest

from residual_binarized_weight_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib

# fake, suitably aligned device addresses: validation must reject before using them
P = ctypes.c_void_p(0x100000)
P_MIS = ctypes.c_void_p(0x100004)   # 4-byte aligned only
P_ODD = ctypes.c_void_p(0x100001)


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "rb.h")).read()
    return sorted(set(re.findall(r"\b(rb_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    syms = declared_symbols()
    assert {"rb_pack", "rb_gemv", "rb_gemm_small", "rb_codebook_encode", "rb_codebook_gemv"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s
        assert s in _lib.SIGNATURES, f"binding lacks {s}"


def test_version_and_status_strings():
    assert L.rb_version() >= 100
    for st in range(6):
        assert L.rb_status_string(st)
    assert L.rb_status_string(0) == b"RB_OK"
    assert L.rb_status_string(99) == b"RB_ERR_UNKNOWN"


def test_storage_bits_per_weight():
    assert L.rb_storage_bits_per_weight(4096, 4096, 2, _lib.RB_F16, 1) == 2.015625
    assert L.rb_storage_bits_per_weight(4096, 4096, 2, _lib.RB_F16, 0) == 2.0 + 16 * 2 * 4096 / 4096 ** 2
    assert L.rb_storage_bits_per_weight(0, 4096, 2, _lib.RB_F16, 1) == -1.0
    assert L.rb_storage_bits_per_weight(16, 16, 5, _lib.RB_F16, 1) == -1.0


def _pack(**kw):
    a = dict(W=P, wdt=_lib.RB_F32, N=16, K=64, ldw=64, k=2, group=0, h=None, sdt=_lib.RB_F16,
             planes=P, ldp=2, g=P, st=None, stream=None)
    a.update(kw)
    return L.rb_pack(a["W"], a["wdt"], a["N"], a["K"], a["ldw"], a["k"], a["group"], a["h"], a["sdt"],
                     a["planes"], a["ldp"], a["g"], a["st"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), _lib.RB_ERR_INVALID_ARG),
    (dict(planes=None), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=0), _lib.RB_ERR_INVALID_ARG),
    (dict(k=0), _lib.RB_ERR_INVALID_ARG),
    (dict(k=5), _lib.RB_ERR_INVALID_ARG),
    (dict(ldw=63), _lib.RB_ERR_INVALID_ARG),
    (dict(ldp=1), _lib.RB_ERR_INVALID_ARG),
    (dict(group=3), _lib.RB_ERR_INVALID_ARG),
    (dict(group=128), _lib.RB_ERR_INVALID_ARG),
    (dict(group=16, h=P), _lib.RB_ERR_UNSUPPORTED),
    (dict(wdt=7), _lib.RB_ERR_INVALID_ARG),
    (dict(sdt=_lib.RB_BF16), _lib.RB_ERR_UNSUPPORTED),
    (dict(planes=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(W=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(st=P_ODD), _lib.RB_ERR_MISALIGNED),
])
def test_pack_rejects(kw, status):
    assert _pack(**kw) == status


def _prod(fn, **kw):
    a = dict(planes=P, ldp=2, g=P, h=None, sdt=_lib.RB_F16, k=2, N=16, K=64, x=P, xdt=_lib.RB_F16, M=1,
             y=P, ydt=_lib.RB_F16, ws=None, wsb=0, stream=None)
    a.update(kw)
    return getattr(L, fn)(a["planes"], a["ldp"], a["g"], a["h"], a["sdt"], a["k"], a["N"], a["K"], a["x"],
                          a["xdt"], a["M"], a["y"], a["ydt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("fn", ["rb_gemv", "rb_gemm_small"])
@pytest.mark.parametrize("kw,status", [
    (dict(planes=None), _lib.RB_ERR_INVALID_ARG),
    (dict(x=None), _lib.RB_ERR_INVALID_ARG),
    (dict(y=None), _lib.RB_ERR_INVALID_ARG),
    (dict(g=None), _lib.RB_ERR_INVALID_ARG),
    (dict(k=0), _lib.RB_ERR_INVALID_ARG),
    (dict(k=5), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(ldp=1), _lib.RB_ERR_INVALID_ARG),
    (dict(xdt=9), _lib.RB_ERR_INVALID_ARG),
    (dict(ydt=_lib.RB_BF16), _lib.RB_ERR_UNSUPPORTED),
    (dict(planes=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(x=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(y=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(h=P_ODD), _lib.RB_ERR_MISALIGNED),
])
def test_product_rejects(fn, kw, status):
    assert _prod(fn, **kw) == status


def test_gemv_batch_limit_and_gemm_constraints():
    assert _prod("rb_gemv", M=17) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", M=4097) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", xdt=_lib.RB_F32) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", K=96, ldp=3) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", K=(1 << 22) + 64, ldp=(1 << 17) + 2) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", ldp=(1 << 20) + 2) == _lib.RB_ERR_UNSUPPORTED
    # h enters the fp16 MFMA operand: fp32 h is refused, and h must be 16-byte aligned
    assert _prod("rb_gemm_small", h=P, sdt=_lib.RB_F32) == _lib.RB_ERR_UNSUPPORTED
    assert _prod("rb_gemm_small", h=ctypes.c_void_p(0x100002)) == _lib.RB_ERR_MISALIGNED


def test_workspace_too_small_is_reported():
    cases = {"rb_gemv": ((2, 4096, 11008, 1), (2, 4096, 4096, 4), (1, 11008, 4096, 16)),
             "rb_gemm_small": ((2, 4096, 4096, 64), (1, 28672, 8192, 64), (2, 28672, 8192, 256))}
    for fn, op in (("rb_gemv", _lib.RB_OP_GEMV), ("rb_gemm_small", _lib.RB_OP_GEMM_SMALL)):
        for (k, N, K, M) in cases[fn]:
            need = L.rb_workspace_bytes(op, k, N, K, M)
            if need == 0:
                continue
            ldp = (K + 31) // 32 + ((K + 31) // 32) % 2
            assert _prod(fn, k=k, N=N, K=K, M=M, ldp=ldp, ws=None, wsb=0) == _lib.RB_ERR_WORKSPACE
            assert _prod(fn, k=k, N=N, K=K, M=M, ldp=ldp, ws=P, wsb=need - 1) == _lib.RB_ERR_WORKSPACE


def zero_region(N):
    return (N * 8 + 255) // 256 * 256


def test_gemv_workspace_holds_the_matrix_core_partials():
    # K a multiple of 64: the zero region (8 bytes per row, 256-byte multiple) and then the
    # matrix-core kernel's K-chunk partials at M = 16, the same size for every M; it is the
    # rb_gemm_small workspace at M = 16 whenever that one splits K
    for (k, N, K) in ((2, 4096, 11008), (1, 512, 4096), (2, 11008, 4096), (2, 28672, 8192)):
        gemm16 = L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, k, N, K, 16)
        for M in (1, 2, 16):
            assert L.rb_workspace_bytes(_lib.RB_OP_GEMV, k, N, K, M) == max(gemm16, zero_region(N))
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 1, 512, 4096, 16) == zero_region(512) + 4 * 16 * 512 * 4
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 28672, 8192, 16) == 0   # no K split
    # other K: the zero region alone
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMV, 2, 300, 1000, 16) == zero_region(300)


def test_scratch_workspaces_start_after_the_zero_region():
    # calls whose workspace is scratch keep clear of the GEMV's zero region, so one buffer
    # serves all calls: each needs the zero region plus its own scratch
    assert L.rb_workspace_bytes(_lib.RB_OP_SVID_INIT, 2, 4096, 11008, 1) > zero_region(4096)
    assert L.rb_workspace_bytes(_lib.RB_OP_QAT_BACKWARD, 2, 4096, 11008, 2048) > zero_region(4096)
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 4096, 11008, 64) > zero_region(4096)


def test_workspace_bytes_invalid_sizes():
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMV, 0, 16, 16, 1) == 0
    assert L.rb_workspace_bytes(_lib.RB_OP_PACK, 2, 16, 16, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(plane=None), _lib.RB_ERR_INVALID_ARG),
    (dict(c=0), _lib.RB_ERR_INVALID_ARG),
    (dict(c=65537), _lib.RB_ERR_INVALID_ARG),
    (dict(v=0), _lib.RB_ERR_INVALID_ARG),
    (dict(v=33), _lib.RB_ERR_INVALID_ARG),
    (dict(ldp=0), _lib.RB_ERR_INVALID_ARG),
    (dict(plane=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(idx=P_ODD), _lib.RB_ERR_MISALIGNED),
])
def test_codebook_encode_rejects(kw, status):
    a = dict(plane=P, ldp=2, N=4, K=64, C=P, c=16, v=20, idx=P, stream=None)
    a.update(kw)
    assert L.rb_codebook_encode(a["plane"], a["ldp"], a["N"], a["K"], a["C"], a["c"], a["v"], a["idx"],
                                a["stream"]) == status


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), _lib.RB_ERR_INVALID_ARG),
    (dict(group=0), _lib.RB_ERR_INVALID_ARG),
    (dict(group=12), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(M=5), _lib.RB_ERR_UNSUPPORTED),
    (dict(c=70000), _lib.RB_ERR_INVALID_ARG),
    (dict(x=P_MIS), _lib.RB_ERR_MISALIGNED),
])
def test_codebook_gemv_rejects(kw, status):
    a = dict(idx=P, C=P, c=16, v=20, s=P, group=16, N=4, K=64, x=P, M=1, y=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    assert L.rb_codebook_gemv(a["idx"], a["C"], a["c"], a["v"], a["s"], a["group"], a["N"], a["K"], a["x"],
                              a["M"], a["y"], a["ws"], a["wsb"], a["stream"]) == status


def _svid(**kw):
    a = dict(W=P, wdt=_lib.RB_F32, N=16, K=64, ldw=64, k=2, T=3, Pi=4, s_in=None, s_out=None, a_in=0.5,
             a_out=0.5, planes=P, ldp=2, g=P, h=P, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.rb_svid_init(a["W"], a["wdt"], a["N"], a["K"], a["ldw"], a["k"], a["T"], a["Pi"], a["s_in"],
                          a["s_out"], a["a_in"], a["a_out"], a["planes"], a["ldp"], a["g"], a["h"], a["ws"],
                          a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), _lib.RB_ERR_INVALID_ARG),
    (dict(planes=None), _lib.RB_ERR_INVALID_ARG),
    (dict(g=None), _lib.RB_ERR_INVALID_ARG),
    (dict(h=None), _lib.RB_ERR_INVALID_ARG),
    (dict(wdt=7), _lib.RB_ERR_INVALID_ARG),
    (dict(wdt=_lib.RB_F16), _lib.RB_ERR_UNSUPPORTED),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=(1 << 28) + 4, ldw=(1 << 28) + 4, ldp=(1 << 23) + 1), _lib.RB_ERR_INVALID_ARG),
    (dict(ldw=63), _lib.RB_ERR_INVALID_ARG),
    (dict(K=62, ldw=62), _lib.RB_ERR_INVALID_ARG),          # row stride not a multiple of 4
    (dict(ldp=1), _lib.RB_ERR_INVALID_ARG),
    (dict(k=0), _lib.RB_ERR_INVALID_ARG),
    (dict(k=5), _lib.RB_ERR_INVALID_ARG),
    (dict(T=0), _lib.RB_ERR_INVALID_ARG),
    (dict(Pi=0), _lib.RB_ERR_INVALID_ARG),
    (dict(Pi=65), _lib.RB_ERR_INVALID_ARG),
    (dict(a_in=float("nan")), _lib.RB_ERR_INVALID_ARG),
    (dict(a_out=float("inf")), _lib.RB_ERR_INVALID_ARG),
    (dict(W=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(planes=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(g=ctypes.c_void_p(0x100002)), _lib.RB_ERR_MISALIGNED),
    (dict(s_in=ctypes.c_void_p(0x100002)), _lib.RB_ERR_MISALIGNED),
    (dict(ws=None), _lib.RB_ERR_WORKSPACE),
    (dict(wsb=16), _lib.RB_ERR_WORKSPACE),
    (dict(ws=P_MIS), _lib.RB_ERR_MISALIGNED),
])
def test_svid_init_rejects(kw, status):
    assert _svid(**kw) == status


def test_svid_workspace_grows_with_the_problem():
    small = L.rb_workspace_bytes(_lib.RB_OP_SVID_INIT, 2, 16, 64, 1)
    assert small > 0
    assert L.rb_workspace_bytes(_lib.RB_OP_SVID_INIT, 2, 4096, 11008, 1) > small
    assert L.rb_workspace_bytes(_lib.RB_OP_SVID_INIT, 3, 16, 64, 1) > small


P2 = ctypes.c_void_p(0x100002)   # 2-byte aligned only


def _qat_derive(**kw):
    a = dict(W=P, N=16, K=64, ldw=64, k=2, g=P, h=P, planes=P, ldp=2, What=P, adt=_lib.RB_BF16, ldwh=64,
             stream=None)
    a.update(kw)
    return L.rb_qat_derive(a["W"], a["N"], a["K"], a["ldw"], a["k"], a["g"], a["h"], a["planes"], a["ldp"],
                           a["What"], a["adt"], a["ldwh"], a["stream"])


def _qat_forward(**kw):
    a = dict(W=P, N=16, K=64, ldw=64, k=2, g=P, h=P, X=P, adt=_lib.RB_F16, M=8, ldx=64, planes=P, ldp=2,
             What=P, ldwh=64, Y=P, ydt=_lib.RB_F32, ldy=16, stream=None)
    a.update(kw)
    return L.rb_qat_forward(a["W"], a["N"], a["K"], a["ldw"], a["k"], a["g"], a["h"], a["X"], a["adt"], a["M"],
                            a["ldx"], a["planes"], a["ldp"], a["What"], a["ldwh"], a["Y"], a["ydt"], a["ldy"],
                            a["stream"])


def _qat_backward(**kw):
    a = dict(dY=P, adt=_lib.RB_BF16, M=8, lddy=16, X=P, ldx=64, What=P, ldwh=64, planes=P, ldp=2, g=P, h=P,
             k=2, N=16, K=64, dW=P, lddw=64, dX=P, dxdt=_lib.RB_F32, lddx=64, dg=P, dh=P, ws=P, wsb=1 << 30,
             stream=None)
    a.update(kw)
    return L.rb_qat_backward(a["dY"], a["adt"], a["M"], a["lddy"], a["X"], a["ldx"], a["What"], a["ldwh"],
                             a["planes"], a["ldp"], a["g"], a["h"], a["k"], a["N"], a["K"], a["dW"], a["lddw"],
                             a["dX"], a["dxdt"], a["lddx"], a["dg"], a["dh"], a["ws"], a["wsb"], a["stream"])


# checks shared by the three training-layer calls
_QAT_COMMON = [
    (dict(g=None), _lib.RB_ERR_INVALID_ARG),
    (dict(h=None), _lib.RB_ERR_INVALID_ARG),
    (dict(planes=None), _lib.RB_ERR_INVALID_ARG),
    (dict(What=None), _lib.RB_ERR_INVALID_ARG),
    (dict(k=0), _lib.RB_ERR_INVALID_ARG),
    (dict(k=5), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=0), _lib.RB_ERR_INVALID_ARG),
    (dict(N=(1 << 28) + 1), _lib.RB_ERR_INVALID_ARG),
    (dict(ldp=1), _lib.RB_ERR_INVALID_ARG),
    (dict(ldwh=63), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=9), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=_lib.RB_F32), _lib.RB_ERR_UNSUPPORTED),
    (dict(g=P2), _lib.RB_ERR_MISALIGNED),
    (dict(h=P2), _lib.RB_ERR_MISALIGNED),
    (dict(planes=P2), _lib.RB_ERR_MISALIGNED),
    (dict(What=P_ODD), _lib.RB_ERR_MISALIGNED),
]


@pytest.mark.parametrize("kw,status", _QAT_COMMON + [
    (dict(W=None), _lib.RB_ERR_INVALID_ARG),
    (dict(ldw=63), _lib.RB_ERR_INVALID_ARG),
    (dict(W=P2), _lib.RB_ERR_MISALIGNED),
])
def test_qat_derive_rejects(kw, status):
    assert _qat_derive(**kw) == status


@pytest.mark.parametrize("kw,status", _QAT_COMMON + [
    (dict(W=None), _lib.RB_ERR_INVALID_ARG),
    (dict(X=None), _lib.RB_ERR_INVALID_ARG),
    (dict(Y=None), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(M=1 << 31), _lib.RB_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(ldy=15), _lib.RB_ERR_INVALID_ARG),
    (dict(ydt=_lib.RB_BF16), _lib.RB_ERR_UNSUPPORTED),   # neither fp32 nor the activation type
    (dict(ydt=5), _lib.RB_ERR_INVALID_ARG),
    (dict(X=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(Y=P2), _lib.RB_ERR_MISALIGNED),                 # fp32 output
])
def test_qat_forward_rejects(kw, status):
    assert _qat_forward(**kw) == status


@pytest.mark.parametrize("kw,status", _QAT_COMMON + [
    (dict(dY=None), _lib.RB_ERR_INVALID_ARG),
    (dict(X=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dW=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dX=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dg=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dh=None), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(lddy=15), _lib.RB_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(lddw=63), _lib.RB_ERR_INVALID_ARG),
    (dict(lddx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(dxdt=_lib.RB_F16), _lib.RB_ERR_UNSUPPORTED),   # activations are bf16 here
    (dict(dY=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(dW=P2), _lib.RB_ERR_MISALIGNED),
    (dict(dg=P2), _lib.RB_ERR_MISALIGNED),
    (dict(ws=None), _lib.RB_ERR_WORKSPACE),
    (dict(wsb=16), _lib.RB_ERR_WORKSPACE),
    (dict(ws=P_MIS), _lib.RB_ERR_MISALIGNED),
])
def test_qat_backward_rejects(kw, status):
    assert _qat_backward(**kw) == status


def test_qat_workspace_covers_the_partial_sums():
    # strips of 256 columns x k x N row partials + tiles of 256 rows x k x K column partials
    ws = L.rb_workspace_bytes(_lib.RB_OP_QAT_BACKWARD, 2, 4096, 11008, 2048) - zero_region(4096)
    assert ws >= 4 * (43 * 2 * 4096 + 16 * 2 * 11008)
    assert ws < 4 * (43 * 2 * 4096 + 16 * 2 * 11008) + 512
    assert L.rb_workspace_bytes(_lib.RB_OP_QAT_BACKWARD, 2, (1 << 28) + 1, 64, 1) == 0


def _qat_autotune(**kw):
    a = dict(X=P, dY=P, adt=_lib.RB_BF16, M=8, ldx=64, lddy=16, What=P, ldwh=64, N=16, K=64, Y=P,
             ydt=_lib.RB_F32, ldy=16, dW=P, lddw=64, dX=P, dxdt=_lib.RB_BF16, lddx=64, stream=None)
    a.update(kw)
    return L.rb_qat_autotune(a["X"], a["dY"], a["adt"], a["M"], a["ldx"], a["lddy"], a["What"], a["ldwh"], a["N"],
                             a["K"], a["Y"], a["ydt"], a["ldy"], a["dW"], a["lddw"], a["dX"], a["dxdt"], a["lddx"],
                             a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dY=None), _lib.RB_ERR_INVALID_ARG),
    (dict(What=None), _lib.RB_ERR_INVALID_ARG),
    (dict(Y=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dW=None), _lib.RB_ERR_INVALID_ARG),
    (dict(dX=None), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=(1 << 28) + 1), _lib.RB_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(lddy=15), _lib.RB_ERR_INVALID_ARG),
    (dict(ldwh=63), _lib.RB_ERR_INVALID_ARG),
    (dict(ldy=15), _lib.RB_ERR_INVALID_ARG),
    (dict(lddw=63), _lib.RB_ERR_INVALID_ARG),
    (dict(lddx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=4), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=_lib.RB_F32), _lib.RB_ERR_UNSUPPORTED),
    (dict(ydt=_lib.RB_F16), _lib.RB_ERR_UNSUPPORTED),
    (dict(dxdt=_lib.RB_F16), _lib.RB_ERR_UNSUPPORTED),
    (dict(X=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(dW=P2), _lib.RB_ERR_MISALIGNED),
])
def test_qat_autotune_rejects(kw, status):
    assert _qat_autotune(**kw) == status


def _qat_matmul(**kw):
    a = dict(X=P, adt=_lib.RB_BF16, M=8, ldx=64, What=P, ldwh=64, N=16, K=64, Y=P, ydt=_lib.RB_F32, ldy=16,
             engine=_lib.RB_QAT_ENGINE_MFMA, stream=None)
    a.update(kw)
    return L.rb_qat_matmul(a["X"], a["adt"], a["M"], a["ldx"], a["What"], a["ldwh"], a["N"], a["K"], a["Y"],
                           a["ydt"], a["ldy"], a["engine"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), _lib.RB_ERR_INVALID_ARG),
    (dict(What=None), _lib.RB_ERR_INVALID_ARG),
    (dict(Y=None), _lib.RB_ERR_INVALID_ARG),
    (dict(M=0), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=0), _lib.RB_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.RB_ERR_INVALID_ARG),
    (dict(ldwh=63), _lib.RB_ERR_INVALID_ARG),
    (dict(ldy=15), _lib.RB_ERR_INVALID_ARG),
    (dict(engine=3), _lib.RB_ERR_INVALID_ARG),
    (dict(engine=-1), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=7), _lib.RB_ERR_INVALID_ARG),
    (dict(adt=_lib.RB_F32), _lib.RB_ERR_UNSUPPORTED),
    (dict(ydt=_lib.RB_F16), _lib.RB_ERR_UNSUPPORTED),   # operands are bf16 here
    (dict(X=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(Y=P2), _lib.RB_ERR_MISALIGNED),
    # the matrix-core engine's layout: 16-byte aligned operands, strides multiples of 8, K of 32
    (dict(K=60, ldx=64, ldwh=64), _lib.RB_ERR_UNSUPPORTED),
    (dict(K=40, ldx=64, ldwh=64), _lib.RB_ERR_UNSUPPORTED),  # a multiple of 8, not of 32
    (dict(ldx=68), _lib.RB_ERR_UNSUPPORTED),
    (dict(ldwh=66), _lib.RB_ERR_UNSUPPORTED),
    (dict(What=P2), _lib.RB_ERR_UNSUPPORTED),
    (dict(M=(1 << 24), ldx=64), _lib.RB_ERR_UNSUPPORTED),     # 2^30 elements of X
])
def test_qat_matmul_rejects(kw, status):
    assert _qat_matmul(**kw) == status


def test_codebook_learn_workspace_bytes():
    # the largest of: a word and a byte per block + 256 chunk counts per 8192 blocks + 256 bucket
    # totals, rounded up to 64 words, + 256 (v + 1) counts per vote slice (the M-step's radix pass
    # and vote), c (v + 1) counters (learning loop), the 2^v-byte map + 2^v-bit bitmap (distinct count)
    blocks = 4096 * 551
    head = -(-(blocks + blocks // 4 + 256 * (-(-blocks // 8192)) + 256) // 64) * 64
    slices = blocks // 4096 + 256
    assert L.rb_codebook_learn_workspace_bytes(4096, 11008, 65536, 20) == 4 * (head + slices * 256 * 21)
    assert L.rb_codebook_learn_workspace_bytes(1, 40, 65536, 20) == 4 * 65536 * 21
    assert L.rb_codebook_learn_workspace_bytes(16, 64, 16, 24) == (1 << 24) + (1 << 21)
    assert L.rb_codebook_learn_workspace_bytes(16, 64, 0, 20) == 0
    assert L.rb_codebook_learn_workspace_bytes(16, 64, 16, 33) == 0
    assert L.rb_codebook_learn_workspace_bytes(0, 64, 16, 20) == 0


def _cb_learn(fn, **kw):
    a = dict(plane=P, ldp=32, N=16, K=1000, v=20, idx=P, C=P, c=256, counts=None, nd=P, iters=2, ws=P,
             wsb=1 << 30, stream=None)
    a.update(kw)
    if fn == "mstep":
        return L.rb_codebook_mstep(a["plane"], a["ldp"], a["N"], a["K"], a["v"], a["idx"], a["C"], a["c"],
                                   a["counts"], a["ws"], a["wsb"], a["stream"])
    if fn == "distinct":
        return L.rb_codebook_distinct(a["plane"], a["ldp"], a["N"], a["K"], a["v"], a["C"], a["c"], a["nd"],
                                      a["ws"], a["wsb"], a["stream"])
    return L.rb_codebook_learn(a["plane"], a["ldp"], a["N"], a["K"], a["v"], a["C"], a["c"], a["iters"], a["idx"],
                               a["nd"], a["ws"], a["wsb"], a["stream"])


_CB_COMMON = [
    (dict(plane=None), _lib.RB_ERR_INVALID_ARG),
    (dict(C=None), _lib.RB_ERR_INVALID_ARG),
    (dict(N=0), _lib.RB_ERR_INVALID_ARG),
    (dict(K=0), _lib.RB_ERR_INVALID_ARG),
    (dict(ldp=31), _lib.RB_ERR_INVALID_ARG),
    (dict(c=0), _lib.RB_ERR_INVALID_ARG),
    (dict(c=65537), _lib.RB_ERR_INVALID_ARG),
    (dict(v=0), _lib.RB_ERR_INVALID_ARG),
    (dict(plane=P_MIS), _lib.RB_ERR_MISALIGNED),
    (dict(C=P2), _lib.RB_ERR_MISALIGNED),
    (dict(ws=None), _lib.RB_ERR_WORKSPACE),
    (dict(wsb=4 * (3 * 256 + 64 + 16 * 50) - 1), _lib.RB_ERR_WORKSPACE),
    (dict(ws=P2), _lib.RB_ERR_MISALIGNED),
]


@pytest.mark.parametrize("kw,status", _CB_COMMON + [
    (dict(idx=None), _lib.RB_ERR_INVALID_ARG),
    (dict(v=33), _lib.RB_ERR_INVALID_ARG),
    (dict(idx=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(counts=P2), _lib.RB_ERR_MISALIGNED),
])
def test_codebook_mstep_rejects(kw, status):
    assert _cb_learn("mstep", **kw) == status


@pytest.mark.parametrize("kw,status", _CB_COMMON + [
    (dict(nd=None), _lib.RB_ERR_INVALID_ARG),
    (dict(v=25), _lib.RB_ERR_INVALID_ARG),
    (dict(nd=P2), _lib.RB_ERR_MISALIGNED),
])
def test_codebook_distinct_rejects(kw, status):
    assert _cb_learn("distinct", **kw) == status


@pytest.mark.parametrize("kw,status", _CB_COMMON + [
    (dict(idx=None), _lib.RB_ERR_INVALID_ARG),
    (dict(nd=None), _lib.RB_ERR_INVALID_ARG),
    (dict(iters=-1), _lib.RB_ERR_INVALID_ARG),
    (dict(iters=1001), _lib.RB_ERR_INVALID_ARG),
    (dict(v=25), _lib.RB_ERR_INVALID_ARG),
    (dict(idx=P_ODD), _lib.RB_ERR_MISALIGNED),
])
def test_codebook_learn_rejects(kw, status):
    assert _cb_learn("learn", **kw) == status


def _gemv_variant(**kw):
    a = dict(planes=P, ldp=2, g=P, h=None, mu=P, zo=0, sdt=_lib.RB_F16, k=2, N=16, K=64, x=P, xdt=_lib.RB_F16, M=1,
             y=P, ydt=_lib.RB_F16, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return L.rb_gemv_variant(a["planes"], a["ldp"], a["g"], a["h"], a["mu"], a["zo"], a["sdt"], a["k"], a["N"],
                             a["K"], a["x"], a["xdt"], a["M"], a["y"], a["ydt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(planes=None), _lib.RB_ERR_INVALID_ARG),
    (dict(g=None), _lib.RB_ERR_INVALID_ARG),
    (dict(zo=2), _lib.RB_ERR_INVALID_ARG),
    (dict(zo=-1), _lib.RB_ERR_INVALID_ARG),
    (dict(k=5), _lib.RB_ERR_INVALID_ARG),
    (dict(M=17), _lib.RB_ERR_UNSUPPORTED),
    (dict(h=P), _lib.RB_ERR_UNSUPPORTED),                  # an offset needs h = 1
    (dict(mu=P_ODD), _lib.RB_ERR_MISALIGNED),
    (dict(mu=P2, sdt=_lib.RB_F32), _lib.RB_ERR_MISALIGNED),
    (dict(h=P_ODD, mu=None), _lib.RB_ERR_MISALIGNED),
    (dict(x=P_MIS), _lib.RB_ERR_MISALIGNED),
])
def test_gemv_variant_rejects(kw, status):
    assert _gemv_variant(**kw) == status


def test_gemm_small_split_workspace():
    # 32 row tiles of the 4096-row layer: K is split in 8 chunks of partial sums (fp32 [8][M][N]);
    # the 28672-row layer fills the GPU with its tiles alone and needs none
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 4096, 11008, 64) == zero_region(4096) + 8 * 64 * 4096 * 4
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 28672, 8192, 256) == 0
    assert L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 4096, 1024, 64) == 0   # chunks < 1024 columns
    need = L.rb_workspace_bytes(_lib.RB_OP_GEMM_SMALL, 2, 4096, 11008, 64)
    assert _prod("rb_gemm_small", k=2, N=4096, K=11008, M=64, ldp=344, ws=P2, wsb=need) == _lib.RB_ERR_MISALIGNED


def test_codebook_table_sizes_and_validation():
    assert L.rb_codebook_table_bytes(20) == (4 << 20) + 128
    assert L.rb_codebook_table_bytes(1) == 8 + 128
    assert L.rb_codebook_table_bytes(25) == 0 and L.rb_codebook_table_bytes(0) == 0
    need = L.rb_codebook_table_bytes(12)

    def call(v=12, ws=P, wsb=None, plane=P, cb=P, idx=P, c=40, N=3, K=100, ldp=4):
        return L.rb_codebook_encode_table(plane, ldp, N, K, cb, c, v, idx, ws, need if wsb is None else wsb, None)
    assert call(plane=None) == _lib.RB_ERR_INVALID_ARG
    # 2^20 rows x 2^17 blocks of 12 columns: 2^37 block positions, past 32 bits
    assert call(N=1 << 20, K=12 << 17, ldp=(12 << 17) // 32) == _lib.RB_ERR_UNSUPPORTED
    assert call(c=0) == _lib.RB_ERR_INVALID_ARG
    assert call(v=33) == _lib.RB_ERR_INVALID_ARG
    assert call(v=25) == _lib.RB_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.RB_ERR_WORKSPACE
    assert call(wsb=need - 1) == _lib.RB_ERR_WORKSPACE
    assert call(idx=ctypes.c_void_p(0x100001)) == _lib.RB_ERR_MISALIGNED
