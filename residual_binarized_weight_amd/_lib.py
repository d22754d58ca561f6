"""ctypes binding of librb (include/rb.h). Argument marshalling only: every step of the
computation runs in the library's HIP kernels. There is no fallback: if librb.so is
missing or fails to load, importing this module raises."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librb.so")

RB_OK, RB_ERR_INVALID_ARG, RB_ERR_UNSUPPORTED, RB_ERR_MISALIGNED, RB_ERR_WORKSPACE, RB_ERR_HIP = range(6)
RB_F32, RB_F16, RB_BF16 = 0, 1, 2
RB_QAT_ENGINE_AUTO, RB_QAT_ENGINE_MFMA, RB_QAT_ENGINE_ROCBLAS = 0, 1, 2
(RB_OP_PACK, RB_OP_GEMV, RB_OP_GEMM_SMALL, RB_OP_CODEBOOK_ENCODE, RB_OP_CODEBOOK_GEMV, RB_OP_SVID_INIT,
 RB_OP_QAT_BACKWARD) = range(7)

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/rb.h
SIGNATURES = {
    "rb_version": (ctypes.c_int, []),
    "rb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "rb_workspace_bytes": (_sz, [ctypes.c_int, _i32, _i64, _i64, _i64]),
    "rb_storage_bits_per_weight": (ctypes.c_double, [_i64, _i64, _i32, ctypes.c_int, _i32]),
    "rb_pack": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _vp, ctypes.c_int,
                               _vp, _i64, _vp, _vp, _vp]),
    "rb_gemv": (ctypes.c_int, [_vp, _i64, _vp, _vp, ctypes.c_int, _i32, _i64, _i64, _vp, ctypes.c_int,
                               _i64, _vp, ctypes.c_int, _vp, _sz, _vp]),
    "rb_gemv_noalloc": (ctypes.c_int, [_vp, _i64, _vp, _vp, ctypes.c_int, _i32, _i64, _i64, _vp, ctypes.c_int,
                                       _i64, _vp, ctypes.c_int, _vp]),
    "rb_gemv_variant": (ctypes.c_int, [_vp, _i64, _vp, _vp, _vp, _i32, ctypes.c_int, _i32, _i64, _i64, _vp,
                                       ctypes.c_int, _i64, _vp, ctypes.c_int, _vp, _sz, _vp]),
    "rb_gemm_small": (ctypes.c_int, [_vp, _i64, _vp, _vp, ctypes.c_int, _i32, _i64, _i64, _vp,
                                     ctypes.c_int, _i64, _vp, ctypes.c_int, _vp, _sz, _vp]),
    "rb_codebook_encode": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _vp]),
    "rb_codebook_gemv": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _i32, _i64, _i64, _vp, _i64, _vp,
                                        _vp, _sz, _vp]),
    "rb_codebook_table_bytes": (_sz, [_i32]),
    "rb_codebook_encode_table": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "rb_codebook_learn_workspace_bytes": (_sz, [_i64, _i64, _i32, _i32]),
    "rb_codebook_mstep": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "rb_codebook_distinct": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "rb_codebook_learn": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "rb_svid_init": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp,
                                    ctypes.c_float, ctypes.c_float, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "rb_qat_derive": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _i64, _vp, ctypes.c_int,
                                     _i64, _vp]),
    "rb_qat_forward": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, ctypes.c_int, _i64, _i64,
                                      _vp, _i64, _vp, _i64, _vp, ctypes.c_int, _i64, _vp]),
    "rb_qat_matmul": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _i64, _i64, _vp, ctypes.c_int, _i64,
                                     _i32, _vp]),
    "rb_qat_backward": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                       _vp, _i32, _i64, _i64, _vp, _i64, _vp, ctypes.c_int, _i64, _vp, _vp,
                                       _vp, _sz, _vp]),
    "rb_qat_autotune": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _i64, _i64, _vp,
                                       ctypes.c_int, _i64, _vp, _i64, _vp, ctypes.c_int, _i64, _vp]),
    # streaming-read probe used by the bench (not part of the method)
    "rb_bench_stream_read": (ctypes.c_int, [_vp, _i64, _vp, _i32, _vp]),
    "rb_bench_gather": (ctypes.c_int, [_vp, ctypes.c_uint32, _i32, _vp, _i32, _vp]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m residual_binarized_weight_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class RbError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.rb_status_string(status).decode()} (status {status})")


def check(fn: str, status: int) -> None:
    if status != RB_OK:
        raise RbError(fn, status)
