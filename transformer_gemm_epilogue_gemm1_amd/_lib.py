"""ctypes view of libcoda.so: the raw C ABI of include/coda.h, nothing else.

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_i64 = ctypes.c_int64
c_vp = ctypes.c_void_p
c_int = ctypes.c_int
c_float = ctypes.c_float
c_size = ctypes.c_size_t
c_double = ctypes.c_double

CODA_BF16 = 0
CODA_F32 = 1

STATUS = {0: "CODA_OK", 1: "CODA_ERR_NULL", 2: "CODA_ERR_SHAPE", 3: "CODA_ERR_ALIGN",
          4: "CODA_ERR_DTYPE", 5: "CODA_ERR_ALIAS", 6: "CODA_ERR_WORKSPACE", 7: "CODA_ERR_HIP"}

# name -> (restype, argtypes), in the order of include/coda.h
SIGNATURES = {
    "coda_prms_num_partials": (c_i64, [c_int, c_i64]),
    "coda_gemm_res_prms": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64,
                                   c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "coda_rms_combine": (c_int, [c_i64, c_i64, c_i64, c_float, c_vp, c_vp, c_vp]),
    "coda_gemm_rowscale": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp,
                                   c_vp, c_i64, c_vp]),
    "coda_packed_bytes": (c_i64, [c_i64, c_i64]),
    "coda_gemm_res_prms_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp,
                                          c_vp, c_i64, c_vp, c_vp, c_vp]),
    "coda_gemm_rowscale_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp]),
    "coda_packed_bytes_e4m3": (c_i64, [c_i64, c_i64]),
    "coda_quantize_cols_e4m3_packed": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp]),
    "coda_quantize_rows_e4m3_packed": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp]),
    "coda_quantize_rows_cols_e4m3_packed": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "coda_quantize_mx_e4m3_packed": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "coda_gemm_res_prms_fp8_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp,
                                              c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "coda_gemm_res_prms_fp8_all_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp,
                                                  c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "coda_gemm_rowscale_fp8_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64,
                                              c_vp]),
    "coda_mx_exp_bytes": (c_i64, [c_i64, c_i64]),
    "coda_gemm_rowscale_swiglu_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp,
                                                 c_i64, c_vp]),
    "coda_gemm_rowscale_lse_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp,
                                              c_vp, c_vp]),
    "coda_gemm_rowscale_ce_bwd_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp,
                                                 c_vp, c_i64, c_vp]),
    "coda_gemm_rowscale_rope_packed": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i64,
                                               c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "coda_gemm_rowscale_swiglu": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp,
                                          c_vp, c_i64, c_vp, c_i64, c_vp]),
    "coda_swiglu_bwd": (c_int, [c_int, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "coda_gemm_rowscale_lse": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, c_vp]),
    "coda_ce_combine": (c_int, [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "coda_gemm_rowscale_ce_bwd": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp,
                                          c_vp, c_vp, c_i64, c_vp]),
    "coda_quantize_rows_e4m3": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "coda_quantize_cols_e4m3": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp]),
    "coda_quantize_rows_cols_e4m3": (c_int, [c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp,
                                             c_vp]),
    "coda_chain_bwd_fp8_workspace_bytes": (c_size, [c_i64, c_i64, c_i64, c_i64]),
    "coda_chain_bwd_fp8": (c_int, [c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                   c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "coda_rope_cache": (c_int, [c_vp, c_i64, c_i64, c_double, c_vp]),
    "coda_gemm_rowscale_rope": (c_int, [c_int, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp,
                                        c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "coda_rope_bwd": (c_int, [c_int, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp,
                              c_i64, c_vp]),
    "coda_gemm_res_prms_fp8": (c_int, [c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_i64,
                                       c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp]),
    "coda_gemm_rowscale_fp8": (c_int, [c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp,
                                       c_i64, c_vp]),
    "coda_ref_chain_workspace_bytes": (c_size, [c_int, c_i64, c_i64]),
    "coda_ref_chain": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64, c_float, c_vp, c_vp, c_vp, c_vp,
                               c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "coda_chain_bwd_workspace_bytes": (c_size, [c_int, c_i64, c_i64, c_i64, c_i64]),
    "coda_chain_bwd": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64,
                               c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                               c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_size, c_vp]),
    "coda_chain_bwd_noalloc": (c_int, [c_int, c_i64, c_i64, c_i64, c_i64,
                                       c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                       c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "coda_status_string": (ctypes.c_char_p, [c_int]),
    "coda_last_error": (ctypes.c_char_p, []),
}

_lib = None


class CodaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def load() -> ctypes.CDLL:
    """The loaded libcoda.so (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libcoda.so not built at {LIB_PATH}: run __graft_entry__.build() "
                          "(python -m transformer_gemm_epilogue_gemm1_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:
            continue  # entry points not yet present are reported by exported_symbols()
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    lib = load()
    return [n for n in SIGNATURES if hasattr(lib, n)]


def check(fn: str, status: int) -> None:
    if status != 0:
        detail = load().coda_last_error().decode()
        raise CodaError(fn, status, detail)
