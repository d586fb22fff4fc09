"""Thin torch-facing binding of libcoda: argument marshalling only.

Each function takes torch tensors on the current HIP device, checks dtype,
device and layout, and passes raw device pointers, leading dimensions and the
current stream to the C entry point of the same name.  All arithmetic runs in
libcoda's kernels; torch only supplies device memory and streams.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.CODA_BF16, torch.float32: _lib.CODA_F32}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")
    return _DT[t.dtype]


def _mat(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> int:
    """Row-major 2-D (or 1-D) device tensor with unit column stride -> leading dim."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dim() == 1:
        if t.numel() > 1 and t.stride(0) != 1:
            raise ValueError(f"{name} must be contiguous")
        return t.shape[0]
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return max(t.stride(0), t.shape[1])


def _dense(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def coda_prms_num_partials(dtype: torch.dtype, D: int) -> int:
    return int(_lib.load().coda_prms_num_partials(_DT[dtype], D))


def coda_gemm_res_prms(A, W1, R, g: Optional[torch.Tensor], H, Hg: Optional[torch.Tensor], partials,
                       stream=None) -> None:
    """H = A W1 + R, Hg = H * g, partial sums of squares of H (see coda.h)."""
    lib = _lib.load()
    dt = A.dtype
    M, K = A.shape
    D = W1.shape[1]
    T = coda_prms_num_partials(dt, D)
    lda = _mat(A, "A", dt, (M, K))
    ldw1 = _mat(W1, "W1", dt, (K, D))
    ldr = _mat(R, "R", dt, (M, D))
    ldh = _mat(H, "H", dt, (M, D))
    ldhg = 0
    if g is not None:
        _mat(g, "g", dt, (D,))
        ldhg = _mat(Hg, "Hg", dt, (M, D))
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    st = lib.coda_gemm_res_prms(_dtype_code(A), M, K, D, A.data_ptr(), lda, W1.data_ptr(), ldw1,
                                R.data_ptr(), ldr, g.data_ptr() if g is not None else None,
                                H.data_ptr(), ldh, Hg.data_ptr() if Hg is not None else None, ldhg,
                                partials.data_ptr(), _stream(stream))
    _lib.check("coda_gemm_res_prms", st)


def coda_rms_combine(partials, r, D: int, eps: float, stream=None) -> None:
    """r_i = 1/sqrt(sum_t partials[t, i] / D + eps)."""
    lib = _lib.load()
    T, M = partials.shape
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    _mat(r, "r", torch.float32, (M,))
    st = lib.coda_rms_combine(M, D, T, float(eps), partials.data_ptr(), r.data_ptr(), _stream(stream))
    _lib.check("coda_rms_combine", st)


def coda_gemm_rowscale(X, W2, r: Optional[torch.Tensor], Y, stream=None) -> None:
    """Y = diag(r) (X W2), the deferred RMSNorm row scale in the epilogue."""
    lib = _lib.load()
    dt = X.dtype
    M, D = X.shape
    N2 = W2.shape[1]
    ldx = _mat(X, "X", dt, (M, D))
    ldw2 = _mat(W2, "W2", dt, (D, N2))
    ldy = _mat(Y, "Y", dt, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale(_dtype_code(X), M, D, N2, X.data_ptr(), ldx, W2.data_ptr(), ldw2,
                                r.data_ptr() if r is not None else None, Y.data_ptr(), ldy,
                                _stream(stream))
    _lib.check("coda_gemm_rowscale", st)


def coda_packed_bytes(rows: int, cols: int) -> int:
    return int(_lib.load().coda_packed_bytes(rows, cols))


def packed_empty(M: int, D: int, device) -> torch.Tensor:
    """A bfloat16 buffer for a tile-packed [M, D] matrix, shaped
    [ceil(M/16), D/8, 16, 8] (row block, column run, row in block, column)."""
    if D % 8 != 0:
        raise ValueError(f"D = {D} must be a multiple of 8")
    return torch.empty(((M + 15) // 16, D // 8, 16, 8), device=device, dtype=torch.bfloat16)


def _packed(Xp: torch.Tensor, name: str, M: int, D: int) -> None:
    if Xp.dtype != torch.bfloat16 or not Xp.is_cuda:
        raise TypeError(f"{name}: expected a bfloat16 CUDA tensor")
    if tuple(Xp.shape) != ((M + 15) // 16, D // 8, 16, 8) or not Xp.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tile-packed buffer of shape "
                         f"{((M + 15) // 16, D // 8, 16, 8)}, got {tuple(Xp.shape)}")


def coda_gemm_res_prms_packed(A, W1, R, g, H, Hgp, partials, stream=None) -> None:
    """coda_gemm_res_prms with Hg written tile-packed into Hgp (packed_empty)."""
    lib = _lib.load()
    dt = A.dtype
    M, K = A.shape
    D = W1.shape[1]
    T = coda_prms_num_partials(dt, D)
    lda = _mat(A, "A", dt, (M, K))
    ldw1 = _mat(W1, "W1", dt, (K, D))
    ldr = _mat(R, "R", dt, (M, D))
    ldh = _mat(H, "H", dt, (M, D))
    _mat(g, "g", dt, (D,))
    _packed(Hgp, "Hg", M, D)
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    st = lib.coda_gemm_res_prms_packed(M, K, D, A.data_ptr(), lda, W1.data_ptr(), ldw1, R.data_ptr(), ldr,
                                       g.data_ptr(), H.data_ptr(), ldh, Hgp.data_ptr(), partials.data_ptr(),
                                       _stream(stream))
    _lib.check("coda_gemm_res_prms_packed", st)


def coda_gemm_rowscale_packed(Xp, W2, r: Optional[torch.Tensor], Y, stream=None) -> None:
    """Y = diag(r) (X W2) with X tile-packed in Xp (as coda_gemm_res_prms_packed writes it)."""
    lib = _lib.load()
    M, N2 = Y.shape
    D = W2.shape[0]
    _packed(Xp, "X", M, D)
    ldw2 = _mat(W2, "W2", torch.bfloat16, (D, N2))
    ldy = _mat(Y, "Y", torch.bfloat16, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_packed(M, D, N2, Xp.data_ptr(), W2.data_ptr(), ldw2,
                                       r.data_ptr() if r is not None else None, Y.data_ptr(), ldy,
                                       _stream(stream))
    _lib.check("coda_gemm_rowscale_packed", st)


def unpack(Xp: torch.Tensor, M: int) -> torch.Tensor:
    """The [M, D] row-major matrix held by a tile-packed buffer (a copy)."""
    nb, nck, _, _ = Xp.shape
    return Xp.permute(0, 2, 1, 3).reshape(nb * 16, nck * 8)[:M]


def coda_gemm_rowscale_swiglu(X, W2, r: Optional[torch.Tensor], Z, Y: Optional[torch.Tensor] = None,
                              stream=None) -> None:
    """Z = silu(Y_gate) * Y_up with Y = diag(r) (X W2), W2 = [W_gate | W_up];
    Y (the pre-activation) is also written when given."""
    lib = _lib.load()
    dt = X.dtype
    M, D = X.shape
    F2 = W2.shape[1]
    if F2 % 2:
        raise ValueError("W2 must have an even number of columns (gate | up)")
    F = F2 // 2
    ldx = _mat(X, "X", dt, (M, D))
    ldw2 = _mat(W2, "W2", dt, (D, F2))
    ldz = _mat(Z, "Z", dt, (M, F))
    ldy = _mat(Y, "Y", dt, (M, F2)) if Y is not None else 0
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_swiglu(_dtype_code(X), M, D, F, X.data_ptr(), ldx, W2.data_ptr(), ldw2,
                                       r.data_ptr() if r is not None else None, Z.data_ptr(), ldz,
                                       Y.data_ptr() if Y is not None else None, ldy, _stream(stream))
    _lib.check("coda_gemm_rowscale_swiglu", st)


def coda_swiglu_bwd(dZ, Y, dY, stream=None) -> None:
    """dY [M, 2F] from dZ [M, F] through Z = silu(Y_gate) * Y_up."""
    lib = _lib.load()
    dt = dZ.dtype
    M, F = dZ.shape
    ldz = _mat(dZ, "dZ", dt, (M, F))
    ldy = _mat(Y, "Y", dt, (M, 2 * F))
    lddy = _mat(dY, "dY", dt, (M, 2 * F))
    st = lib.coda_swiglu_bwd(_dtype_code(dZ), M, F, dZ.data_ptr(), ldz, Y.data_ptr(), ldy, dY.data_ptr(), lddy,
                             _stream(stream))
    _lib.check("coda_swiglu_bwd", st)


def coda_gemm_rowscale_lse(X, Wv, r: Optional[torch.Tensor], targets, pmax, psum, tgt, stream=None) -> None:
    """LM-head GEMM writing the cross-entropy statistics (per-tile max and
    sum-exp of y = diag(r) X Wv, and the target logit) instead of the logits."""
    lib = _lib.load()
    dt = X.dtype
    M, D = X.shape
    V = Wv.shape[1]
    T = coda_prms_num_partials(dt, V)
    ldx = _mat(X, "X", dt, (M, D))
    ldw = _mat(Wv, "Wv", dt, (D, V))
    _mat(targets, "targets", torch.int32, (M,))
    for t, n in ((pmax, "pmax"), (psum, "psum")):
        _mat(t, n, torch.float32, (T, M))
        _dense(t, n)
    _mat(tgt, "tgt", torch.float32, (M,))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_lse(_dtype_code(X), M, D, V, X.data_ptr(), ldx, Wv.data_ptr(), ldw,
                                    r.data_ptr() if r is not None else None, targets.data_ptr(), pmax.data_ptr(),
                                    psum.data_ptr(), tgt.data_ptr(), _stream(stream))
    _lib.check("coda_gemm_rowscale_lse", st)


def rope_cache(max_pos: int, d_head: int, base: float = 10000.0, device="cuda", stream=None) -> torch.Tensor:
    """The rotary table [max_pos, d_head // 2, 2] (cos, sin) of coda_rope_cache."""
    cs = torch.empty((max_pos, d_head // 2, 2), device=device, dtype=torch.float32)
    st = _lib.load().coda_rope_cache(cs.data_ptr(), max_pos, d_head, float(base), _stream(stream))
    _lib.check("coda_rope_cache", st)
    return cs


def _rope_args(positions, cos_sin, M: int, d_head: int):
    _mat(positions, "positions", torch.int32, (M,))
    if not isinstance(cos_sin, torch.Tensor) or cos_sin.dim() != 3 or tuple(cos_sin.shape[1:]) != (d_head // 2, 2):
        raise ValueError(f"cos_sin must be the [max_pos, {d_head // 2}, 2] table of rope_cache")
    if cos_sin.dtype != torch.float32 or cos_sin.device.type != "cuda":
        raise TypeError("cos_sin must be a float32 device tensor")
    _dense(cos_sin, "cos_sin")
    return cos_sin.shape[0]


def coda_gemm_rowscale_rope(X, Wqkv, r: Optional[torch.Tensor], positions, cos_sin, n_q: int, n_k: int,
                            d_head: int, Y, stream=None) -> None:
    """Y = rope(diag(r) X Wqkv): the QKV projection with the rotary embedding
    applied to its first n_q + n_k columns (heads of d_head)."""
    lib = _lib.load()
    dt = X.dtype
    M, D = X.shape
    N2 = Wqkv.shape[1]
    ldx = _mat(X, "X", dt, (M, D))
    ldw = _mat(Wqkv, "Wqkv", dt, (D, N2))
    ldy = _mat(Y, "Y", dt, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    max_pos = _rope_args(positions, cos_sin, M, d_head)
    st = lib.coda_gemm_rowscale_rope(_dtype_code(X), M, D, N2, X.data_ptr(), ldx, Wqkv.data_ptr(), ldw,
                                     r.data_ptr() if r is not None else None, positions.data_ptr(),
                                     cos_sin.data_ptr(), max_pos, n_q, n_k, d_head, Y.data_ptr(), ldy,
                                     _stream(stream))
    _lib.check("coda_gemm_rowscale_rope", st)


def coda_rope_bwd(dYr, positions, cos_sin, n_q: int, n_k: int, d_head: int, dY, stream=None) -> None:
    """dY = the gradient dYr of the rotated projection turned back by RoPE."""
    lib = _lib.load()
    dt = dYr.dtype
    M, N2 = dYr.shape
    ldg = _mat(dYr, "dYr", dt, (M, N2))
    lddy = _mat(dY, "dY", dt, (M, N2))
    max_pos = _rope_args(positions, cos_sin, M, d_head)
    st = lib.coda_rope_bwd(_dtype_code(dYr), M, N2, dYr.data_ptr(), ldg, positions.data_ptr(), cos_sin.data_ptr(),
                           max_pos, n_q, n_k, d_head, dY.data_ptr(), lddy, _stream(stream))
    _lib.check("coda_rope_bwd", st)


def coda_gemm_rowscale_ce_bwd(X, Wv, r: Optional[torch.Tensor], targets, lse, dloss, dY, stream=None) -> None:
    """dY = dloss * (softmax(diag(r) X Wv) - onehot(targets)): the gradient of
    the per-token losses with respect to the logits, recomputed from X."""
    lib = _lib.load()
    dt = X.dtype
    M, D = X.shape
    V = Wv.shape[1]
    ldx = _mat(X, "X", dt, (M, D))
    ldw = _mat(Wv, "Wv", dt, (D, V))
    lddy = _mat(dY, "dY", dt, (M, V))
    _mat(targets, "targets", torch.int32, (M,))
    _mat(lse, "lse", torch.float32, (M,))
    _mat(dloss, "dloss", torch.float32, (M,))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_ce_bwd(_dtype_code(X), M, D, V, X.data_ptr(), ldx, Wv.data_ptr(), ldw,
                                       r.data_ptr() if r is not None else None, targets.data_ptr(), lse.data_ptr(),
                                       dloss.data_ptr(), dY.data_ptr(), lddy, _stream(stream))
    _lib.check("coda_gemm_rowscale_ce_bwd", st)


def coda_ce_combine(pmax, psum, tgt, targets, lse, loss, V: int, stream=None) -> None:
    """lse and per-token loss from the LM-head statistics."""
    lib = _lib.load()
    T, M = pmax.shape
    for t, n in ((pmax, "pmax"), (psum, "psum")):
        _mat(t, n, torch.float32, (T, M))
        _dense(t, n)
    for t, n in ((tgt, "tgt"), (lse, "lse"), (loss, "loss")):
        _mat(t, n, torch.float32, (M,))
    _mat(targets, "targets", torch.int32, (M,))
    st = lib.coda_ce_combine(M, V, T, pmax.data_ptr(), psum.data_ptr(), tgt.data_ptr(), targets.data_ptr(),
                             lse.data_ptr(), loss.data_ptr(), _stream(stream))
    _lib.check("coda_ce_combine", st)


_FP8 = (torch.uint8, getattr(torch, "float8_e4m3fn", torch.uint8))


def _mat8(t: torch.Tensor, name: str, shape) -> int:
    """e4m3 operand: torch.float8_e4m3fn (OCP e4m3) or raw uint8 codes."""
    if t.dtype not in _FP8:
        raise TypeError(f"{name} has dtype {t.dtype}, expected float8_e4m3fn or uint8 e4m3 codes")
    return _mat(t, name, t.dtype, shape)


def _mx_shape(rows: int, cols: int):
    return ((cols + 255) // 256, (rows + 127) // 128, 2, 32, 4, 4)


def mx_exp_empty(rows: int, cols: int, device) -> torch.Tensor:
    """A block-exponent array for a [rows, cols] MX operand: uint8
    [G, B, 2, 32, 4, 4] with G = ceil(cols / 256) groups of 4 k-tiles and
    B = ceil(rows / 128) row blocks; byte [t // 4, i // 128, h, i % 32,
    (i // 32) % 4, t % 4] is the E8M0 exponent of columns [64 t + 32 h, + 32)
    of row i (the rows past `rows` in the last block are padding)."""
    return torch.empty(_mx_shape(rows, cols), device=device, dtype=torch.uint8)


def mx_exponents_of(E: torch.Tensor, rows: int, cols: int) -> torch.Tensor:
    """The int32 exponents [rows, ceil(cols / 32)] an exponent array holds
    (E8M0 codes minus 127); block b of a row is half b % 2 of k-tile b // 2."""
    nb = (cols + 31) // 32
    b = torch.arange(nb, device=E.device)
    t = b // 2
    i = torch.arange(rows, device=E.device)
    return E[(t // 4)[None, :], (i // 128)[:, None], (b % 2)[None, :], (i % 32)[:, None], ((i // 32) % 4)[:, None],
             (t % 4)[None, :]].to(torch.int32) - 127


def _mx(E: torch.Tensor, name: str, rows: int, cols: int) -> None:
    shape = _mx_shape(rows, cols)
    if E.dtype != torch.uint8 or tuple(E.shape) != shape or not E.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous uint8 tensor of shape {shape}, got {E.dtype} {tuple(E.shape)}")
    if E.data_ptr() % 16 != 0:
        raise ValueError(f"{name} is not 16-byte aligned")


def coda_gemm_res_prms_fp8(A8, sa, W1t8, sw1, R, g, H, Hg8, Hg8_exp, partials, stream=None) -> None:
    """fp8 first GEMM: H = bf16(acc sa sw1 + R), Hg8 = e4m3(H g 2^-E) with the
    MX block exponents E in Hg8_exp (mx_exp_empty(M, D)), partial sums of squares."""
    lib = _lib.load()
    M, K = A8.shape
    D = W1t8.shape[0]
    T = coda_prms_num_partials(torch.bfloat16, D)
    lda = _mat8(A8, "A8", (M, K))
    ldw = _mat8(W1t8, "W1t8", (D, K))
    ldhg = _mat8(Hg8, "Hg8", (M, D))
    _mx(Hg8_exp, "Hg8_exp", M, D)
    _mat(sa, "sa", torch.float32, (M,))
    _mat(sw1, "sw1", torch.float32, (D,))
    ldr = _mat(R, "R", torch.bfloat16, (M, D))
    _mat(g, "g", torch.bfloat16, (D,))
    ldh = _mat(H, "H", torch.bfloat16, (M, D))
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    st = lib.coda_gemm_res_prms_fp8(M, K, D, A8.data_ptr(), lda, sa.data_ptr(), W1t8.data_ptr(), ldw,
                                    sw1.data_ptr(), R.data_ptr(), ldr, g.data_ptr(), H.data_ptr(), ldh,
                                    Hg8.data_ptr(), ldhg, Hg8_exp.data_ptr(), partials.data_ptr(), _stream(stream))
    _lib.check("coda_gemm_res_prms_fp8", st)


def coda_gemm_rowscale_fp8(X8, X8_exp: Optional[torch.Tensor], W2t8, sw2, r: Optional[torch.Tensor], Y,
                           stream=None) -> None:
    """fp8 second GEMM: Y = bf16(acc r sw2), acc over X8's codes times 2^E
    (X8_exp, or E = 0 when None), W2 given transposed ([N2, D])."""
    lib = _lib.load()
    M, D = X8.shape
    N2 = W2t8.shape[0]
    ldx = _mat8(X8, "X8", (M, D))
    ldw = _mat8(W2t8, "W2t8", (N2, D))
    if X8_exp is not None:
        _mx(X8_exp, "X8_exp", M, D)
    _mat(sw2, "sw2", torch.float32, (N2,))
    ldy = _mat(Y, "Y", torch.bfloat16, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_fp8(M, D, N2, X8.data_ptr(), ldx, X8_exp.data_ptr() if X8_exp is not None else None,
                                    W2t8.data_ptr(), ldw, sw2.data_ptr(),
                                    r.data_ptr() if r is not None else None, Y.data_ptr(), ldy, _stream(stream))
    _lib.check("coda_gemm_rowscale_fp8", st)


def coda_ref_chain_workspace_bytes(dtype: torch.dtype, M: int, D: int) -> int:
    return int(_lib.load().coda_ref_chain_workspace_bytes(_DT[dtype], M, D))


def coda_ref_chain(A, W1, R, g, W2, H, r, Y, ws, eps: float, stream=None) -> None:
    """Unfused chain: GEMM, residual add, RMSNorm, GEMM (all dense tensors)."""
    lib = _lib.load()
    dt = A.dtype
    M, K = A.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    for t, n, dtp, shp in ((A, "A", dt, (M, K)), (W1, "W1", dt, (K, D)), (R, "R", dt, (M, D)),
                           (g, "g", dt, (D,)), (W2, "W2", dt, (D, N2)), (H, "H", dt, (M, D)),
                           (r, "r", torch.float32, (M,)), (Y, "Y", dt, (M, N2))):
        _mat(t, n, dtp, shp)
        _dense(t, n)
    if ws.device.type != "cuda":
        raise ValueError("workspace must be on a HIP device")
    st = lib.coda_ref_chain(_dtype_code(A), M, K, D, N2, float(eps), A.data_ptr(), W1.data_ptr(),
                            R.data_ptr(), g.data_ptr(), W2.data_ptr(), H.data_ptr(), r.data_ptr(),
                            Y.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream))
    _lib.check("coda_ref_chain", st)


def coda_chain_bwd_workspace_bytes(dtype: torch.dtype, M: int, K: int, D: int, N2: int) -> int:
    return int(_lib.load().coda_chain_bwd_workspace_bytes(_DT[dtype], M, K, D, N2))


def coda_chain_bwd(dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg, ws, stream=None) -> None:
    """Backward of the chain: dA, dR (= dH), dW1, dW2, dg from dY and the
    forward's stored H and r (all dense tensors; see coda.h)."""
    lib = _lib.load()
    dt = A.dtype
    M, K = A.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    for t, n, dtp, shp in ((dY, "dY", dt, (M, N2)), (A, "A", dt, (M, K)), (W1, "W1", dt, (K, D)),
                           (g, "g", dt, (D,)), (W2, "W2", dt, (D, N2)), (H, "H", dt, (M, D)),
                           (r, "r", torch.float32, (M,)), (dA, "dA", dt, (M, K)), (dR, "dR", dt, (M, D)),
                           (dW1, "dW1", dt, (K, D)), (dW2, "dW2", dt, (D, N2)),
                           (dg, "dg", torch.float32, (D,))):
        _mat(t, n, dtp, shp)
        _dense(t, n)
    if ws.device.type != "cuda":
        raise ValueError("workspace must be on a HIP device")
    st = lib.coda_chain_bwd(_dtype_code(A), M, K, D, N2, dY.data_ptr(), A.data_ptr(), W1.data_ptr(),
                            g.data_ptr(), W2.data_ptr(), H.data_ptr(), r.data_ptr(), dA.data_ptr(),
                            dR.data_ptr(), dW1.data_ptr(), dW2.data_ptr(), dg.data_ptr(), ws.data_ptr(),
                            ws.numel() * ws.element_size(), _stream(stream))
    _lib.check("coda_chain_bwd", st)


def coda_chain_bwd_noalloc(dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg, stream=None) -> None:
    """coda_chain_bwd without a workspace: the library's static scratch holds
    X_n, the partial sums and c (see coda.h for the size limit).  For callers
    that cannot allocate; calls that overlap on one GPU race on the scratch."""
    lib = _lib.load()
    dt = A.dtype
    M, K = A.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    for t, n, dtp, shp in ((dY, "dY", dt, (M, N2)), (A, "A", dt, (M, K)), (W1, "W1", dt, (K, D)),
                           (g, "g", dt, (D,)), (W2, "W2", dt, (D, N2)), (H, "H", dt, (M, D)),
                           (r, "r", torch.float32, (M,)), (dA, "dA", dt, (M, K)), (dR, "dR", dt, (M, D)),
                           (dW1, "dW1", dt, (K, D)), (dW2, "dW2", dt, (D, N2)),
                           (dg, "dg", torch.float32, (D,))):
        _mat(t, n, dtp, shp)
        _dense(t, n)
    st = lib.coda_chain_bwd_noalloc(_dtype_code(A), M, K, D, N2, dY.data_ptr(), A.data_ptr(), W1.data_ptr(),
                                    g.data_ptr(), W2.data_ptr(), H.data_ptr(), r.data_ptr(), dA.data_ptr(),
                                    dR.data_ptr(), dW1.data_ptr(), dW2.data_ptr(), dg.data_ptr(), _stream(stream))
    _lib.check("coda_chain_bwd_noalloc", st)


# ---- conveniences that allocate outputs with torch, then call the above ----

def fused_forward(A, W1, R, g, W2, eps: float, stream=None):
    """The fused chain: three launches, returns (H, Hg, r, Y, partials)."""
    M, D, N2 = A.shape[0], W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hg = torch.empty((M, D), device=dev, dtype=dt)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=dt)
    coda_gemm_res_prms(A, W1, R, g, H, Hg, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale(Hg, W2, r, Y, stream)
    return H, Hg, r, Y, P


def fused_forward_packed(A, W1, R, g, W2, eps: float, stream=None):
    """The fused chain with Hg tile-packed between the two GEMMs: returns
    (H, Hgp, r, Y, partials); Hgp as packed_empty (unpack gives Hg)."""
    M, D, N2 = A.shape[0], W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hgp = packed_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=dt)
    coda_gemm_res_prms_packed(A, W1, R, g, H, Hgp, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_packed(Hgp, W2, r, Y, stream)
    return H, Hgp, r, Y, P


def ref_chain(A, W1, R, g, W2, eps: float, stream=None):
    """The unfused chain, returns (H, r, Y)."""
    M, D, N2 = A.shape[0], W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=dt)
    ws = torch.empty((coda_ref_chain_workspace_bytes(dt, M, D),), device=dev, dtype=torch.uint8)
    coda_ref_chain(A, W1, R, g, W2, H, r, Y, ws, eps, stream)
    return H, r, Y


def fused_backward(dY, A, W1, g, W2, H, r, stream=None):
    """Backward of the chain, returns (dA, dR, dW1, dW2, dg); dR = dH."""
    M, K = A.shape
    D, N2 = W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    dA = torch.empty((M, K), device=dev, dtype=dt)
    dR = torch.empty((M, D), device=dev, dtype=dt)
    dW1 = torch.empty((K, D), device=dev, dtype=dt)
    dW2 = torch.empty((D, N2), device=dev, dtype=dt)
    dg = torch.empty((D,), device=dev, dtype=torch.float32)
    ws = torch.empty((coda_chain_bwd_workspace_bytes(dt, M, K, D, N2),), device=dev, dtype=torch.uint8)
    coda_chain_bwd(dY, A, W1, g, W2, H, r, dA, dR, dW1, dW2, dg, ws, stream)
    return dA, dR, dW1, dW2, dg


def fused_forward_swiglu(A, W1, R, g, W2, eps: float, keep_y: bool = False, stream=None):
    """The fused chain with the SwiGLU gate in the second GEMM's epilogue:
    returns (H, Hg, r, Z, Y) with Y None unless keep_y."""
    M, D, F2 = A.shape[0], W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hg = torch.empty((M, D), device=dev, dtype=dt)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Z = torch.empty((M, F2 // 2), device=dev, dtype=dt)
    Y = torch.empty((M, F2), device=dev, dtype=dt) if keep_y else None
    coda_gemm_res_prms(A, W1, R, g, H, Hg, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_swiglu(Hg, W2, r, Z, Y, stream)
    return H, Hg, r, Z, Y


def coda_gemm_rowscale_swiglu_packed(Xp, W2, r: Optional[torch.Tensor], Z, Y: Optional[torch.Tensor] = None,
                                     stream=None) -> None:
    """coda_gemm_rowscale_swiglu with X tile-packed in Xp (as coda_gemm_res_prms_packed writes it)."""
    lib = _lib.load()
    M, F = Z.shape
    D, F2 = W2.shape
    if F2 != 2 * F:
        raise ValueError("W2 must have 2F columns (gate | up)")
    _packed(Xp, "X", M, D)
    ldw2 = _mat(W2, "W2", torch.bfloat16, (D, F2))
    ldz = _mat(Z, "Z", torch.bfloat16, (M, F))
    ldy = _mat(Y, "Y", torch.bfloat16, (M, F2)) if Y is not None else 0
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_swiglu_packed(M, D, F, Xp.data_ptr(), W2.data_ptr(), ldw2,
                                              r.data_ptr() if r is not None else None, Z.data_ptr(), ldz,
                                              Y.data_ptr() if Y is not None else None, ldy, _stream(stream))
    _lib.check("coda_gemm_rowscale_swiglu_packed", st)


def fused_forward_swiglu_packed(A, W1, R, g, W2, eps: float, keep_y: bool = False, stream=None):
    """fused_forward_swiglu with Hg tile-packed between the GEMMs: returns
    (H, Hgp, r, Z, Y) with Y None unless keep_y."""
    M, D, F2 = A.shape[0], W1.shape[1], W2.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hgp = packed_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Z = torch.empty((M, F2 // 2), device=dev, dtype=dt)
    Y = torch.empty((M, F2), device=dev, dtype=dt) if keep_y else None
    coda_gemm_res_prms_packed(A, W1, R, g, H, Hgp, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_swiglu_packed(Hgp, W2, r, Z, Y, stream)
    return H, Hgp, r, Z, Y


def fused_backward_swiglu(dZ, Y, A, W1, g, W2, H, r, stream=None):
    """Backward of the chain with the SwiGLU gate: dY through the gate, then
    the chain's backward; returns (dA, dR, dW1, dW2, dg, dY)."""
    dY = torch.empty_like(Y)
    coda_swiglu_bwd(dZ, Y, dY, stream)
    return fused_backward(dY, A, W1, g, W2, H, r, stream) + (dY,)


def quantize_rows_e4m3(X, stream=None, X8=None, scales=None):
    """Per-row e4m3 codes (uint8 [M, K]) and float32 scales of a bf16 X,
    into X8 / scales when given."""
    M, K = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, K))
    if X8 is None:
        X8 = torch.empty((M, K), device=X.device, dtype=torch.uint8)
    if scales is None:
        scales = torch.empty((M,), device=X.device, dtype=torch.float32)
    ldx8 = _mat(X8, "X8", torch.uint8, (M, K))
    _mat(scales, "scales", torch.float32, (M,))
    sc = scales
    st = _lib.load().coda_quantize_rows_e4m3(M, K, X.data_ptr(), ldx, X8.data_ptr(), ldx8, sc.data_ptr(),
                                             _stream(stream))
    _lib.check("coda_quantize_rows_e4m3", st)
    return X8, sc


def quantize_weight_e4m3(W, stream=None, Wt8=None, scales=None):
    """Transposed e4m3 codes (uint8 [N, K]) and per-output-channel float32
    scales of a bf16 weight W [K, N], into Wt8 / scales when given."""
    K, N = W.shape
    ldw = _mat(W, "W", torch.bfloat16, (K, N))
    if Wt8 is None:
        Wt8 = torch.empty((N, K), device=W.device, dtype=torch.uint8)
    if scales is None:
        scales = torch.empty((N,), device=W.device, dtype=torch.float32)
    ldwt = _mat(Wt8, "Wt8", torch.uint8, (N, K))
    _mat(scales, "scales", torch.float32, (N,))
    sc = scales
    st = _lib.load().coda_quantize_cols_e4m3(K, N, W.data_ptr(), ldw, Wt8.data_ptr(), ldwt, sc.data_ptr(),
                                             _stream(stream))
    _lib.check("coda_quantize_cols_e4m3", st)
    return Wt8, sc


def packed_empty_e4m3(rows: int, cols: int, device) -> torch.Tensor:
    """A uint8 buffer for a tile-packed e4m3 [rows, cols] matrix, shaped
    [ceil(rows/16), cols/16, 16, 16] (row block, 16-code run, row in block, code)."""
    if cols % 16 != 0:
        raise ValueError(f"cols = {cols} must be a multiple of 16")
    return torch.empty(((rows + 15) // 16, cols // 16, 16, 16), device=device, dtype=torch.uint8)


def _packed8(Xp: torch.Tensor, name: str, rows: int, cols: int) -> None:
    if Xp.dtype not in _FP8 or not Xp.is_cuda:
        raise TypeError(f"{name}: expected a uint8 / float8_e4m3fn CUDA tensor")
    if tuple(Xp.shape) != ((rows + 15) // 16, cols // 16, 16, 16) or not Xp.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tile-packed buffer of shape "
                         f"{((rows + 15) // 16, cols // 16, 16, 16)}, got {tuple(Xp.shape)}")


def quantize_weight_e4m3_packed(W, stream=None, Wt8p=None, scales=None):
    """quantize_weight_e4m3 with the transposed codes [N, K] written
    tile-packed (packed_empty_e4m3(N, K)); returns (Wt8p, scales)."""
    K, N = W.shape
    ldw = _mat(W, "W", torch.bfloat16, (K, N))
    if Wt8p is None:
        Wt8p = packed_empty_e4m3(N, K, W.device)
    if scales is None:
        scales = torch.empty((N,), device=W.device, dtype=torch.float32)
    _packed8(Wt8p, "Wt8", N, K)
    _mat(scales, "scales", torch.float32, (N,))
    st = _lib.load().coda_quantize_cols_e4m3_packed(K, N, W.data_ptr(), ldw, Wt8p.data_ptr(), scales.data_ptr(),
                                                    _stream(stream))
    _lib.check("coda_quantize_cols_e4m3_packed", st)
    return Wt8p, scales


def coda_gemm_res_prms_fp8_packed(A8, sa, W1t8, sw1, R, g, H, Hg8p, Hg8_exp, partials, stream=None) -> None:
    """coda_gemm_res_prms_fp8 with Hg8 written tile-packed into Hg8p."""
    lib = _lib.load()
    M, K = A8.shape
    D = W1t8.shape[0]
    T = coda_prms_num_partials(torch.bfloat16, D)
    lda = _mat8(A8, "A8", (M, K))
    ldw = _mat8(W1t8, "W1t8", (D, K))
    _packed8(Hg8p, "Hg8", M, D)
    _mx(Hg8_exp, "Hg8_exp", M, D)
    _mat(sa, "sa", torch.float32, (M,))
    _mat(sw1, "sw1", torch.float32, (D,))
    ldr = _mat(R, "R", torch.bfloat16, (M, D))
    _mat(g, "g", torch.bfloat16, (D,))
    ldh = _mat(H, "H", torch.bfloat16, (M, D))
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    st = lib.coda_gemm_res_prms_fp8_packed(M, K, D, A8.data_ptr(), lda, sa.data_ptr(), W1t8.data_ptr(), ldw,
                                           sw1.data_ptr(), R.data_ptr(), ldr, g.data_ptr(), H.data_ptr(), ldh,
                                           Hg8p.data_ptr(), Hg8_exp.data_ptr(), partials.data_ptr(),
                                           _stream(stream))
    _lib.check("coda_gemm_res_prms_fp8_packed", st)


def coda_gemm_res_prms_fp8_all_packed(A8p, sa, W1t8p, sw1, R, g, H, Hg8p, Hg8_exp, partials, stream=None) -> None:
    """coda_gemm_res_prms_fp8_packed with A8p (packed_empty_e4m3(M, K), as
    quantize_rows_e4m3_packed writes it) and W1t8p (packed_empty_e4m3(D, K), as
    quantize_weight_e4m3_packed writes it) tile-packed too; M and D from R."""
    lib = _lib.load()
    M, D = R.shape
    K = 16 * A8p.shape[1]
    T = coda_prms_num_partials(torch.bfloat16, D)
    _packed8(A8p, "A8p", M, K)
    _packed8(W1t8p, "W1t8p", D, K)
    _packed8(Hg8p, "Hg8", M, D)
    _mx(Hg8_exp, "Hg8_exp", M, D)
    _mat(sa, "sa", torch.float32, (M,))
    _mat(sw1, "sw1", torch.float32, (D,))
    ldr = _mat(R, "R", torch.bfloat16, (M, D))
    _mat(g, "g", torch.bfloat16, (D,))
    ldh = _mat(H, "H", torch.bfloat16, (M, D))
    _mat(partials, "partials", torch.float32, (T, M))
    _dense(partials, "partials")
    st = lib.coda_gemm_res_prms_fp8_all_packed(M, K, D, A8p.data_ptr(), sa.data_ptr(), W1t8p.data_ptr(),
                                               sw1.data_ptr(), R.data_ptr(), ldr, g.data_ptr(), H.data_ptr(), ldh,
                                               Hg8p.data_ptr(), Hg8_exp.data_ptr(), partials.data_ptr(),
                                               _stream(stream))
    _lib.check("coda_gemm_res_prms_fp8_all_packed", st)


def coda_gemm_rowscale_fp8_packed(X8p, X8_exp: Optional[torch.Tensor], W2t8p, sw2, r: Optional[torch.Tensor], Y,
                                  stream=None) -> None:
    """coda_gemm_rowscale_fp8 with both operands tile-packed (X8_exp row-major)."""
    lib = _lib.load()
    M, N2 = Y.shape
    D = X8p.shape[1] * 16
    _packed8(X8p, "X8", M, D)
    _packed8(W2t8p, "W2t8", N2, D)
    if X8_exp is not None:
        _mx(X8_exp, "X8_exp", M, D)
    _mat(sw2, "sw2", torch.float32, (N2,))
    ldy = _mat(Y, "Y", torch.bfloat16, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_fp8_packed(M, D, N2, X8p.data_ptr(),
                                           X8_exp.data_ptr() if X8_exp is not None else None,
                                           W2t8p.data_ptr(), sw2.data_ptr(),
                                           r.data_ptr() if r is not None else None, Y.data_ptr(), ldy,
                                           _stream(stream))
    _lib.check("coda_gemm_rowscale_fp8_packed", st)


def unpack_e4m3(Xp: torch.Tensor, rows: int) -> torch.Tensor:
    """The [rows, cols] row-major codes held by a tile-packed e4m3 buffer (a copy)."""
    nb, nck, _, _ = Xp.shape
    return Xp.permute(0, 2, 1, 3).reshape(nb * 16, nck * 16)[:rows]


def fused_forward_fp8_packed(A8, sa, W1t8, sw1, R, g, W2t8p, sw2, eps: float, stream=None):
    """The fp8 chain with Hg8 and W2t8 tile-packed: returns (H, Hg8p, Hg8_exp, r, Y, partials)."""
    M, D, N2 = A8.shape[0], W1t8.shape[0], sw2.shape[0]
    dev = A8.device
    H = torch.empty((M, D), device=dev, dtype=torch.bfloat16)
    Hg8p = packed_empty_e4m3(M, D, dev)
    E = mx_exp_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(torch.bfloat16, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=torch.bfloat16)
    coda_gemm_res_prms_fp8_packed(A8, sa, W1t8, sw1, R, g, H, Hg8p, E, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_fp8_packed(Hg8p, E, W2t8p, sw2, r, Y, stream)
    return H, Hg8p, E, r, Y, P


def fused_forward_fp8_all_packed(A8p, sa, W1t8p, sw1, R, g, W2t8p, sw2, eps: float, stream=None):
    """The fp8 chain with every e4m3 operand tile-packed (A8p, W1t8p, Hg8,
    W2t8p): returns (H, Hg8p, Hg8_exp, r, Y, partials)."""
    M, D = R.shape
    N2 = sw2.shape[0]
    dev = R.device
    H = torch.empty((M, D), device=dev, dtype=torch.bfloat16)
    Hg8p = packed_empty_e4m3(M, D, dev)
    E = mx_exp_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(torch.bfloat16, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=torch.bfloat16)
    coda_gemm_res_prms_fp8_all_packed(A8p, sa, W1t8p, sw1, R, g, H, Hg8p, E, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_fp8_packed(Hg8p, E, W2t8p, sw2, r, Y, stream)
    return H, Hg8p, E, r, Y, P


def quantize_rows_cols_e4m3(X, stream=None):
    """Both e4m3 quantisations of a bf16 activation X [M, N]: the row codes
    (uint8 [M, N]) with their scales [M], and the transposed column codes
    (uint8 [N, M]) with their scales [N]."""
    M, N = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, N))
    X8 = torch.empty((M, N), device=X.device, dtype=torch.uint8)
    Xt8 = torch.empty((N, M), device=X.device, dtype=torch.uint8)
    sr = torch.empty((M,), device=X.device, dtype=torch.float32)
    sc = torch.empty((N,), device=X.device, dtype=torch.float32)
    st = _lib.load().coda_quantize_rows_cols_e4m3(M, N, X.data_ptr(), ldx, X8.data_ptr(), N, sr.data_ptr(),
                                                  Xt8.data_ptr(), M, sc.data_ptr(), _stream(stream))
    _lib.check("coda_quantize_rows_cols_e4m3", st)
    return X8, sr, Xt8, sc


def quantize_rows_e4m3_packed(X, stream=None, X8p=None, scales=None):
    """quantize_rows_e4m3 with the codes [M, K] written tile-packed
    (packed_empty_e4m3(M, K)), into X8p / scales when given; returns
    (X8p, scales)."""
    M, K = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, K))
    if X8p is None:
        X8p = packed_empty_e4m3(M, K, X.device)
    _packed8(X8p, "X8p", M, K)
    sc = torch.empty((M,), device=X.device, dtype=torch.float32) if scales is None else scales
    _mat(sc, "scales", torch.float32, (M,))
    st = _lib.load().coda_quantize_rows_e4m3_packed(M, K, X.data_ptr(), ldx, X8p.data_ptr(), sc.data_ptr(),
                                                    _stream(stream))
    _lib.check("coda_quantize_rows_e4m3_packed", st)
    return X8p, sc


def quantize_rows_cols_e4m3_packed(X, stream=None):
    """quantize_rows_cols_e4m3 with both code arrays tile-packed: returns
    (X8p [M, N] packed, row scales, Xt8p [N, M] packed, column scales)."""
    M, N = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, N))
    X8p = packed_empty_e4m3(M, N, X.device)
    Xt8p = packed_empty_e4m3(N, M, X.device)
    sr = torch.empty((M,), device=X.device, dtype=torch.float32)
    sc = torch.empty((N,), device=X.device, dtype=torch.float32)
    st = _lib.load().coda_quantize_rows_cols_e4m3_packed(M, N, X.data_ptr(), ldx, X8p.data_ptr(), sr.data_ptr(),
                                                         Xt8p.data_ptr(), sc.data_ptr(), _stream(stream))
    _lib.check("coda_quantize_rows_cols_e4m3_packed", st)
    return X8p, sr, Xt8p, sc


def quantize_mx_e4m3_packed(X, rows: bool = True, cols: bool = True, stream=None):
    """MX e4m3 codes of a bf16 X [M, N] with one block exponent per 32
    elements: along the rows (Xr8p [M, N] tile-packed, Er = mx_exp_empty(M,
    N)) and / or along the columns (the codes of X^T, Xc8p [N, M] tile-packed,
    Ec = mx_exp_empty(N, M)).  Returns (Xr8p, Er, Xc8p, Ec), None for a pair
    not asked for."""
    if not (rows or cols):
        raise ValueError("ask for the row codes, the column codes or both")
    M, N = X.shape
    ldx = _mat(X, "X", torch.bfloat16, (M, N))
    dev = X.device
    Xr8p, Er = (packed_empty_e4m3(M, N, dev), mx_exp_empty(M, N, dev)) if rows else (None, None)
    Xc8p, Ec = (packed_empty_e4m3(N, M, dev), mx_exp_empty(N, M, dev)) if cols else (None, None)
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = _lib.load().coda_quantize_mx_e4m3_packed(M, N, X.data_ptr(), ldx, ptr(Xr8p), ptr(Er), ptr(Xc8p), ptr(Ec),
                                                  _stream(stream))
    _lib.check("coda_quantize_mx_e4m3_packed", st)
    return Xr8p, Er, Xc8p, Ec


def fused_forward_fp8(A8, sa, W1t8, sw1, R, g, W2t8, sw2, eps: float, stream=None):
    """The fused chain with fp8 GEMM operands: returns (H, Hg8, Hg8_exp, r, Y,
    partials), Hg8_exp the MX block exponents of Hg8 (mx_exp_empty layout)."""
    M, D, N2 = A8.shape[0], W1t8.shape[0], W2t8.shape[0]
    dev = A8.device
    H = torch.empty((M, D), device=dev, dtype=torch.bfloat16)
    Hg8 = torch.empty((M, D), device=dev, dtype=A8.dtype)
    E = mx_exp_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(torch.bfloat16, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=torch.bfloat16)
    coda_gemm_res_prms_fp8(A8, sa, W1t8, sw1, R, g, H, Hg8, E, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_fp8(Hg8, E, W2t8, sw2, r, Y, stream)
    return H, Hg8, E, r, Y, P


def fused_forward_ce(A, W1, R, g, Wv, eps: float, targets, stream=None):
    """The chain ending in the LM head and the per-token cross-entropy:
    returns (H, Hg, r, lse, loss); the logits are never materialised."""
    M, D, V = A.shape[0], W1.shape[1], Wv.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hg = torch.empty((M, D), device=dev, dtype=dt)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    T = coda_prms_num_partials(dt, V)
    pmax = torch.empty((T, M), device=dev, dtype=torch.float32)
    psum = torch.empty((T, M), device=dev, dtype=torch.float32)
    tgt = torch.empty((M,), device=dev, dtype=torch.float32)
    lse = torch.empty((M,), device=dev, dtype=torch.float32)
    loss = torch.empty((M,), device=dev, dtype=torch.float32)
    coda_gemm_res_prms(A, W1, R, g, H, Hg, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_lse(Hg, Wv, r, targets, pmax, psum, tgt, stream)
    coda_ce_combine(pmax, psum, tgt, targets, lse, loss, V, stream)
    return H, Hg, r, lse, loss


def fused_backward_ce(A, W1, g, Wv, H, Hg, r, targets, lse, dloss, stream=None):
    """Backward of the chain ending in the cross-entropy head: dY from the
    recomputed logits, then the chain's backward; returns
    (dA, dR, dW1, dWv, dg, dY)."""
    dY = torch.empty((A.shape[0], Wv.shape[1]), device=A.device, dtype=A.dtype)
    coda_gemm_rowscale_ce_bwd(Hg, Wv, r, targets, lse, dloss, dY, stream)
    return fused_backward(dY, A, W1, g, Wv, H, r, stream) + (dY,)


def fused_forward_rope(A, W1, R, g, Wqkv, eps: float, positions, cos_sin, n_q: int, n_k: int, d_head: int,
                       stream=None):
    """The chain whose second GEMM is the QKV projection with RoPE: returns
    (H, Hg, r, Y) with Y the rotated [Q | K | V]."""
    M, D, N2 = A.shape[0], W1.shape[1], Wqkv.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hg = torch.empty((M, D), device=dev, dtype=dt)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=dt)
    coda_gemm_res_prms(A, W1, R, g, H, Hg, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_rope(Hg, Wqkv, r, positions, cos_sin, n_q, n_k, d_head, Y, stream)
    return H, Hg, r, Y


def coda_gemm_rowscale_lse_packed(Xp, Wv, r: Optional[torch.Tensor], targets, pmax, psum, tgt,
                                  stream=None) -> None:
    """coda_gemm_rowscale_lse with X tile-packed in Xp (as coda_gemm_res_prms_packed writes it)."""
    lib = _lib.load()
    M = targets.shape[0]
    D, V = Wv.shape
    T = coda_prms_num_partials(torch.bfloat16, V)
    _packed(Xp, "X", M, D)
    ldw = _mat(Wv, "Wv", torch.bfloat16, (D, V))
    _mat(targets, "targets", torch.int32, (M,))
    for t, n in ((pmax, "pmax"), (psum, "psum")):
        _mat(t, n, torch.float32, (T, M))
        _dense(t, n)
    _mat(tgt, "tgt", torch.float32, (M,))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_lse_packed(M, D, V, Xp.data_ptr(), Wv.data_ptr(), ldw,
                                           r.data_ptr() if r is not None else None, targets.data_ptr(),
                                           pmax.data_ptr(), psum.data_ptr(), tgt.data_ptr(), _stream(stream))
    _lib.check("coda_gemm_rowscale_lse_packed", st)


def coda_gemm_rowscale_ce_bwd_packed(Xp, Wv, r: Optional[torch.Tensor], targets, lse, dloss, dY,
                                     stream=None) -> None:
    """coda_gemm_rowscale_ce_bwd with X tile-packed in Xp (as coda_gemm_res_prms_packed writes it)."""
    lib = _lib.load()
    M = dY.shape[0]
    D, V = Wv.shape
    _packed(Xp, "X", M, D)
    ldw = _mat(Wv, "Wv", torch.bfloat16, (D, V))
    lddy = _mat(dY, "dY", torch.bfloat16, (M, V))
    _mat(targets, "targets", torch.int32, (M,))
    _mat(lse, "lse", torch.float32, (M,))
    _mat(dloss, "dloss", torch.float32, (M,))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    st = lib.coda_gemm_rowscale_ce_bwd_packed(M, D, V, Xp.data_ptr(), Wv.data_ptr(), ldw,
                                              r.data_ptr() if r is not None else None, targets.data_ptr(),
                                              lse.data_ptr(), dloss.data_ptr(), dY.data_ptr(), lddy,
                                              _stream(stream))
    _lib.check("coda_gemm_rowscale_ce_bwd_packed", st)


def coda_gemm_rowscale_rope_packed(Xp, Wqkv, r: Optional[torch.Tensor], positions, cos_sin, n_q: int, n_k: int,
                                   d_head: int, Y, stream=None) -> None:
    """coda_gemm_rowscale_rope with X tile-packed in Xp (as coda_gemm_res_prms_packed writes it)."""
    lib = _lib.load()
    M, N2 = Y.shape
    D = Wqkv.shape[0]
    _packed(Xp, "X", M, D)
    ldw = _mat(Wqkv, "Wqkv", torch.bfloat16, (D, N2))
    ldy = _mat(Y, "Y", torch.bfloat16, (M, N2))
    if r is not None:
        _mat(r, "r", torch.float32, (M,))
    max_pos = _rope_args(positions, cos_sin, M, d_head)
    st = lib.coda_gemm_rowscale_rope_packed(M, D, N2, Xp.data_ptr(), Wqkv.data_ptr(), ldw,
                                            r.data_ptr() if r is not None else None, positions.data_ptr(),
                                            cos_sin.data_ptr(), max_pos, n_q, n_k, d_head, Y.data_ptr(), ldy,
                                            _stream(stream))
    _lib.check("coda_gemm_rowscale_rope_packed", st)


def fused_forward_ce_packed(A, W1, R, g, Wv, eps: float, targets, stream=None):
    """fused_forward_ce with Hg tile-packed between the GEMMs: returns
    (H, Hgp, r, lse, loss)."""
    M, D, V = A.shape[0], W1.shape[1], Wv.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hgp = packed_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    T = coda_prms_num_partials(dt, V)
    pmax = torch.empty((T, M), device=dev, dtype=torch.float32)
    psum = torch.empty((T, M), device=dev, dtype=torch.float32)
    tgt = torch.empty((M,), device=dev, dtype=torch.float32)
    lse = torch.empty((M,), device=dev, dtype=torch.float32)
    loss = torch.empty((M,), device=dev, dtype=torch.float32)
    coda_gemm_res_prms_packed(A, W1, R, g, H, Hgp, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_lse_packed(Hgp, Wv, r, targets, pmax, psum, tgt, stream)
    coda_ce_combine(pmax, psum, tgt, targets, lse, loss, V, stream)
    return H, Hgp, r, lse, loss


def fused_backward_ce_packed(A, W1, g, Wv, H, Hgp, r, targets, lse, dloss, stream=None):
    """fused_backward_ce reading the tile-packed Hgp of fused_forward_ce_packed."""
    dY = torch.empty((A.shape[0], Wv.shape[1]), device=A.device, dtype=A.dtype)
    coda_gemm_rowscale_ce_bwd_packed(Hgp, Wv, r, targets, lse, dloss, dY, stream)
    return fused_backward(dY, A, W1, g, Wv, H, r, stream) + (dY,)


def fused_forward_rope_packed(A, W1, R, g, Wqkv, eps: float, positions, cos_sin, n_q: int, n_k: int, d_head: int,
                              stream=None):
    """fused_forward_rope with Hg tile-packed between the GEMMs: returns
    (H, Hgp, r, Y)."""
    M, D, N2 = A.shape[0], W1.shape[1], Wqkv.shape[1]
    dev, dt = A.device, A.dtype
    H = torch.empty((M, D), device=dev, dtype=dt)
    Hgp = packed_empty(M, D, dev)
    P = torch.empty((coda_prms_num_partials(dt, D), M), device=dev, dtype=torch.float32)
    r = torch.empty((M,), device=dev, dtype=torch.float32)
    Y = torch.empty((M, N2), device=dev, dtype=dt)
    coda_gemm_res_prms_packed(A, W1, R, g, H, Hgp, P, stream)
    coda_rms_combine(P, r, D, eps, stream)
    coda_gemm_rowscale_rope_packed(Hgp, Wqkv, r, positions, cos_sin, n_q, n_k, d_head, Y, stream)
    return H, Hgp, r, Y


def fused_forward_fp8_from_bf16(A, W1t8, sw1, R, g, W2t8, sw2, eps: float, stream=None):
    """The fp8 chain fed with a bf16 activation A: A quantised per row on the
    device, then the fp8 chain; returns (H, Hg8, Hg8_exp, r, Y, partials, A8, sa)."""
    A8, sa = quantize_rows_e4m3(A, stream)
    return fused_forward_fp8(A8, sa, W1t8, sw1, R, g, W2t8, sw2, eps, stream) + (A8, sa)


def fused_backward_fp8(dY, A, W1, g, W2, H, r, stream=None):
    """Backward of the chain with e4m3 products (coda_chain_bwd_fp8), bf16
    tensors in and out; returns (dA, dR, dW1, dW2, dg)."""
    lib = _lib.load()
    M, K = A.shape
    D, N2 = W1.shape[1], W2.shape[1]
    bf = torch.bfloat16
    for t, n, shp in ((dY, "dY", (M, N2)), (A, "A", (M, K)), (W1, "W1", (K, D)), (g, "g", (D,)), (W2, "W2", (D, N2)),
                      (H, "H", (M, D))):
        _mat(t, n, bf, shp)
        _dense(t, n)
    _mat(r, "r", torch.float32, (M,))
    dev = A.device
    dA = torch.empty((M, K), device=dev, dtype=bf)
    dR = torch.empty((M, D), device=dev, dtype=bf)
    dW1 = torch.empty((K, D), device=dev, dtype=bf)
    dW2 = torch.empty((D, N2), device=dev, dtype=bf)
    dg = torch.empty((D,), device=dev, dtype=torch.float32)
    nbytes = int(lib.coda_chain_bwd_fp8_workspace_bytes(M, K, D, N2))
    ws = torch.empty((max(nbytes, 256),), device=dev, dtype=torch.uint8)
    st = lib.coda_chain_bwd_fp8(M, K, D, N2, dY.data_ptr(), A.data_ptr(), W1.data_ptr(), g.data_ptr(), W2.data_ptr(),
                                H.data_ptr(), r.data_ptr(), dA.data_ptr(), dR.data_ptr(), dW1.data_ptr(),
                                dW2.data_ptr(), dg.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
    _lib.check("coda_chain_bwd_fp8", st)
    return dA, dR, dW1, dW2, dg
