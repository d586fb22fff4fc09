"""libcoda: the fused GEMM-Residual-PartialRMS-GEMM chain and its backward on AMD MI355X (gfx950).

The HIP kernels and the C ABI live in csrc/ and include/coda.h; this package
is a thin binding over libcoda.so.  Importing it loads the library and fails
if it has not been built.
"""
from . import _lib
from ._lib import CodaError
from .binding import (coda_ce_combine, coda_chain_bwd, coda_chain_bwd_workspace_bytes,  # noqa: F401
                      coda_chain_bwd_noalloc,
                      coda_gemm_res_prms, coda_gemm_rowscale_lse, fused_forward_ce,
                      coda_gemm_res_prms_fp8, coda_gemm_rowscale, coda_gemm_rowscale_fp8,
                      coda_gemm_rowscale_swiglu, coda_prms_num_partials, coda_ref_chain,
                      coda_ref_chain_workspace_bytes, coda_rms_combine, coda_swiglu_bwd, fused_backward,
                      fused_backward_swiglu, fused_forward, fused_forward_fp8, fused_forward_swiglu, ref_chain,
                      coda_gemm_rowscale_rope, coda_rope_bwd, fused_forward_rope, rope_cache,
                      coda_gemm_rowscale_ce_bwd, fused_backward_ce,
                      fused_forward_fp8_from_bf16, quantize_rows_e4m3, quantize_weight_e4m3,
                      quantize_rows_cols_e4m3, fused_backward_fp8, quantize_rows_e4m3_packed,
                      quantize_rows_cols_e4m3_packed,
                      coda_packed_bytes, packed_empty, unpack, coda_gemm_res_prms_packed,
                      coda_gemm_rowscale_packed, fused_forward_packed,
                      packed_empty_e4m3, unpack_e4m3, quantize_weight_e4m3_packed,
                      coda_gemm_res_prms_fp8_packed, coda_gemm_rowscale_fp8_packed, fused_forward_fp8_packed,
                      coda_gemm_rowscale_swiglu_packed, fused_forward_swiglu_packed,
                      coda_gemm_rowscale_lse_packed, coda_gemm_rowscale_ce_bwd_packed, coda_gemm_rowscale_rope_packed,
                      fused_forward_ce_packed, fused_backward_ce_packed, fused_forward_rope_packed,
                      mx_exp_empty, mx_exponents_of, quantize_mx_e4m3_packed,
                      coda_gemm_res_prms_fp8_all_packed, fused_forward_fp8_all_packed)

_lib.load()
