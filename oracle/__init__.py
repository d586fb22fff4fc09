"""CPU fp64 oracle for the GEMM-Residual-RMSNorm-GEMM chain (its SwiGLU epilogue, fp8 variant, cross-entropy head and RoPE projection).

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its Python binding.
"""
from .chain import backward, forward  # noqa: F401
from .swiglu import backward_swiglu, forward_swiglu, silu, swiglu_dy  # noqa: F401
from .fp8 import (backward_fp8, bf16_round, e4m3_decode, e4m3_encode, forward_fp8, mx_dequantize,  # noqa: F401
                  mx_exponents, mx_quantize, quantize_cols_transposed, quantize_rows)
from .ce import backward_ce, cross_entropy_grad, cross_entropy_rows, forward_ce, logsumexp_rows  # noqa: F401
from .rope import forward_rope, rope_angles, rope_backward, rope_rotate  # noqa: F401
