"""Seeded synthetic inputs for the GEMM-Residual-PartialRMS-GEMM chain.

This module is the one piece shared by the CPU oracle's tests and the GPU
path's tests and benchmark.  It only draws random numbers and quantises them
to the storage dtype; it holds none of the chain's arithmetic.

Workloads are LLaMA-shaped: M tokens, a hidden size D, an input width K
(K = D: the first GEMM is a square projection) and N2 = 2F output columns
of the second GEMM (gate and up projections side by side).

Value recipe (every workload):
    A, R ~ N(0, 1)                     activations and residual stream
    W1 ~ N(0, 1/K), W2 ~ N(0, 1/D)     variance 1 / (contraction length)
    g  = 1 + 0.1 * N(0, 1)             RMSNorm weight
    dY ~ N(0, 1)                       upstream gradient (backward only)
drawn in float32 from numpy's PCG64 seeded by SeedSequence([seed, wl_id,
tensor_id]), then rounded to nearest-even bfloat16 for the bf16 workloads.

fp8 workloads (make_inputs_fp8) draw the same values and store A, W1 and W2
as OCP e4m3 codes with float32 scales: A per row, W1 and W2 per output
channel, each scale = (max |value| over the scaled vector) / 448, the
weights transposed to [N, K] (contraction contiguous).  R and g stay bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

# tensor ids inside one workload's seed sequence
TENSOR_IDS = {"A": 0, "R": 1, "W1": 2, "W2": 3, "g": 4, "dY": 5, "targets": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wl_id: int
    M: int
    K: int
    D: int
    N2: int
    eps: float
    dtype: str  # "f32" or "bf16"
    backward: bool = False

    @property
    def fwd_flops(self) -> float:
        return 2.0 * self.M * self.K * self.D + 2.0 * self.M * self.D * self.N2

    @property
    def bwd_flops(self) -> float:
        return 2.0 * self.fwd_flops


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        # tiny fp32 parity case: one small projection + 2x-wide second GEMM
        Workload("tiny-fp32", 0, 256, 256, 256, 512, 1e-6, "f32"),
        # 1B-style hidden size 2048, FFN 8192 (gate||up = 16384), 8 x 2048 tokens
        Workload("1b-bf16", 1, 16384, 2048, 2048, 16384, 1e-5, "bf16"),
        # 7B-style hidden size 4096, FFN 14336 (gate||up = 28672), 8 x 2048 tokens
        Workload("7b-bf16", 2, 16384, 4096, 4096, 28672, 1e-5, "bf16"),
        # 70B hidden size 8192, FFN 28672 (gate||up = 57344), 4 x 2048 tokens
        Workload("70b-bf16", 3, 8192, 8192, 8192, 57344, 1e-5, "bf16"),
        # backward of the 7B-style chain
        Workload("7b-bwd-bf16", 4, 16384, 4096, 4096, 28672, 1e-5, "bf16", True),
        # 7B-style chain with fp8 (e4m3) GEMM operands
        Workload("7b-fp8", 5, 16384, 4096, 4096, 28672, 1e-5, "fp8"),
        # 7B-style chain ending in the LM head (vocabulary 32000) and the
        # per-token cross-entropy
        Workload("7b-ce-bf16", 6, 16384, 4096, 4096, 32000, 1e-5, "bf16"),
        # 7B-style chain whose second GEMM is the attention QKV projection
        # (32 query, 32 key and 32 value heads of 128) with RoPE
        Workload("7b-rope-bf16", 7, 16384, 4096, 4096, 12288, 1e-5, "bf16"),
    ]
}


def custom_workload(M: int, K: int, D: int, N2: int, eps: float = 1e-5,
                    dtype: str = "bf16", wl_id: int = 100,
                    name: Optional[str] = None) -> Workload:
    """A workload with the same value recipe at an arbitrary shape."""
    return Workload(name or f"custom-{M}x{K}x{D}x{N2}-{dtype}", wl_id, M, K, D,
                    N2, eps, dtype)


def generator(seed: int, wl_id: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, wl_id, TENSOR_IDS[tensor]])))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(seed: int, wl: Workload, tensor: str, shape, std: float, mean: float = 0.0):
    g = generator(seed, wl.wl_id, tensor)
    x = g.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


class HostTensor:
    """A host array in its storage dtype plus its exact float32 value view.

    bits: uint16 bf16 patterns (bf16) or float32 values (f32) - what the GPU gets
    f32:  the same values as float32 (exact widening)
    """

    def __init__(self, values_f32: np.ndarray, dtype: str):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = bf16_bits(values_f32)
            self.f32 = bf16_bits_to_f32(self.bits)
        elif dtype == "f32":
            self.bits = np.ascontiguousarray(values_f32, dtype=np.float32)
            self.f32 = self.bits
        else:
            raise ValueError(dtype)

    @property
    def shape(self):
        return self.f32.shape

    def f64(self) -> np.ndarray:
        return self.f32.astype(np.float64)


def make_inputs(wl: Workload, seed: int = 0, with_dy: Optional[bool] = None) -> Dict[str, HostTensor]:
    """All inputs of one workload: A[M,K], R[M,D], W1[K,D], W2[D,N2], g[D] (+ dY[M,N2])."""
    M, K, D, N2 = wl.M, wl.K, wl.D, wl.N2
    out = {
        "A": HostTensor(_draw(seed, wl, "A", (M, K), 1.0), wl.dtype),
        "R": HostTensor(_draw(seed, wl, "R", (M, D), 1.0), wl.dtype),
        "W1": HostTensor(_draw(seed, wl, "W1", (K, D), 1.0 / np.sqrt(K)), wl.dtype),
        "W2": HostTensor(_draw(seed, wl, "W2", (D, N2), 1.0 / np.sqrt(D)), wl.dtype),
        "g": HostTensor(_draw(seed, wl, "g", (D,), 0.1, 1.0), wl.dtype),
    }
    if with_dy if with_dy is not None else wl.backward:
        out["dY"] = HostTensor(_draw(seed, wl, "dY", (M, N2), 1.0), wl.dtype)
    return out


# ---- fp8 (OCP e4m3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
# largest finite 448, no infinities, S.1111.111 is NaN) ----

E4M3_MAX = 448.0


def e4m3_values(codes: np.ndarray) -> np.ndarray:
    """Exact float32 values of e4m3 codes (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int32)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag).astype(np.float32)


def e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even e4m3 codes, saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # spacing of the representable values around a: 2^(e - 3), subnormals 2^-9
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = np.exp2(e - 3.0)
    q = np.round(a / step) * step            # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    eq = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    norm = q >= 2.0 ** -6
    code = np.where(norm, ((eq + 7).astype(np.int64) << 3) + (q / np.exp2(eq - 3.0) - 8).astype(np.int64),
                    (q / 2.0 ** -9).astype(np.int64))
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _quantize_rows(x: np.ndarray):
    """Per-row e4m3 codes and float32 scales: scale = max|row| / 448."""
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    return e4m3_codes(x / scale[:, None]), scale


def make_inputs_fp8(wl: Workload, seed: int = 0) -> Dict[str, object]:
    """fp8 inputs of one workload (same draws as make_inputs):
    A8[M,K] codes + sa[M]; W1t8[D,K] codes (W1 transposed) + sw1[D];
    W2t8[N2,D] codes (W2 transposed) + sw2[N2]; R[M,D], g[D] bf16."""
    M, K, D, N2 = wl.M, wl.K, wl.D, wl.N2
    A8, sa = _quantize_rows(_draw(seed, wl, "A", (M, K), 1.0))
    W1t8, sw1 = _quantize_rows(np.ascontiguousarray(_draw(seed, wl, "W1", (K, D), 1.0 / np.sqrt(K)).T))
    W2t8, sw2 = _quantize_rows(np.ascontiguousarray(_draw(seed, wl, "W2", (D, N2), 1.0 / np.sqrt(D)).T))
    return {"A8": A8, "sa": sa, "W1t8": W1t8, "sw1": sw1, "W2t8": W2t8, "sw2": sw2,
            "R": HostTensor(_draw(seed, wl, "R", (M, D), 1.0), "bf16"),
            "g": HostTensor(_draw(seed, wl, "g", (D,), 0.1, 1.0), "bf16")}


def make_targets(wl: Workload, seed: int = 0) -> np.ndarray:
    """One target class per row, uniform over the N2 (vocabulary) columns, int32."""
    return generator(seed, wl.wl_id, "targets").integers(0, wl.N2, size=wl.M).astype(np.int32)


def make_positions(wl: Workload, seq_len: int = 2048) -> np.ndarray:
    """Token positions of the rows: M / seq_len sequences of seq_len tokens
    (position = row mod seq_len), int32."""
    return (np.arange(wl.M) % seq_len).astype(np.int32)
