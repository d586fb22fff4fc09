"""The C ABI on the host (CPU only): libcoda loads, exports every function that
include/coda.h declares, and rejects bad arguments before touching the GPU.

Pointers below are fake, 16-byte aligned addresses: every call here fails
validation (or is a documented no-op), so nothing is ever dereferenced or
enqueued.  Also builds and runs the g++ check of the kernels' index maps.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")

from transformer_gemm_epilogue_gemm1_amd import _lib  # noqa: E402

OK, NULL, SHAPE, ALIGN, DTYPE, ALIAS, WS, HIP = range(8)
BF16, F32 = 0, 1
P = 0x7F0000000000  # fake device addresses, far apart
A_, W1_, R_, G_, H_, HG_, PART_, W2_, Y_, R2_, WS_, DY_, DA_, DR_, DW1_, DW2_, DG_, EX_ = (
    P + i * (1 << 36) for i in range(18))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "coda_gemm_res_prms" in names and "coda_rms_combine" in names
    assert "coda_gemm_rowscale" in names and "coda_ref_chain" in names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared in coda.h but not exported: {missing}"
    unknown = [n for n in names if n not in _lib.SIGNATURES]
    assert not unknown, f"binding lacks signatures for {unknown}"


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert lib.coda_status_string(code).decode() == name
    assert lib.coda_status_string(99).decode() == "CODA_ERR_UNKNOWN"


def test_num_partials_and_workspace(lib):
    # one partial per 64 columns, whole 256-column tiles
    assert lib.coda_prms_num_partials(BF16, 4096) == 64
    assert lib.coda_prms_num_partials(BF16, 2048) == 32
    assert lib.coda_prms_num_partials(F32, 8) == 4
    assert lib.coda_prms_num_partials(BF16, 264) == 8
    assert lib.coda_prms_num_partials(5, 64) == -1
    assert lib.coda_prms_num_partials(BF16, 0) == -1
    c = ((16384 * 4096 * 4 + 255) // 256) * 256
    assert lib.coda_ref_chain_workspace_bytes(BF16, 16384, 4096) == c + 16384 * 4096 * 2
    assert lib.coda_ref_chain_workspace_bytes(F32, 3, 8) == 256 + 3 * 8 * 4


def prms(lib, dt=BF16, M=512, K=256, D=512, A=A_, lda=None, W1=W1_, ldw1=None, R=R_, ldr=None, g=G_,
         H=H_, ldh=None, Hg=HG_, ldhg=None, part=PART_):
    return lib.coda_gemm_res_prms(dt, M, K, D, A, lda or K, W1, ldw1 or D, R, ldr or D, g, H, ldh or D,
                                  Hg, ldhg or D, part, None)


def rowscale(lib, dt=BF16, M=512, D=256, N2=512, X=H_, ldx=None, W2=W2_, ldw2=None, r=R2_, Y=Y_, ldy=None):
    return lib.coda_gemm_rowscale(dt, M, D, N2, X, ldx or D, W2, ldw2 or N2, r, Y, ldy or N2, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), DTYPE),
    (dict(M=-1), SHAPE),
    (dict(K=0), SHAPE),
    (dict(K=252), SHAPE),
    (dict(D=100), SHAPE),
    (dict(A=None), NULL),
    (dict(W1=None), NULL),
    (dict(R=None), NULL),
    (dict(H=None), NULL),
    (dict(part=None), NULL),
    (dict(g=None), NULL),          # g and Hg must come together
    (dict(Hg=None), NULL),
    (dict(A=A_ + 8), ALIGN),
    (dict(lda=260), ALIGN),        # ld not a multiple of 8 elements
    (dict(lda=128), SHAPE),        # ld < K
    (dict(ldh=256), SHAPE),        # ld < D
    (dict(H=A_), ALIAS),
    (dict(Hg=H_ + 64), ALIAS),
    (dict(part=R_ + 4096), ALIAS),
    (dict(M=1 << 31), SHAPE),
    (dict(M=1 << 20, K=4096, lda=4096 * 1024), SHAPE),  # A spans more than 2 GiB
])
def test_gemm_res_prms_rejects(lib, kw, status):
    assert prms(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


def test_gemm_res_prms_empty_is_noop(lib):
    assert prms(lib, M=0, A=None, R=None, H=None, part=None) == OK
    assert lib.coda_last_error().decode() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(dt=9), DTYPE),
    (dict(N2=12), SHAPE),
    (dict(X=None), NULL),
    (dict(W2=W2_ + 4), ALIGN),
    (dict(ldy=256), SHAPE),
    (dict(Y=H_), ALIAS),
    (dict(Y=R2_), ALIAS),
    (dict(r=R2_ + 2), ALIGN),
])
def test_gemm_rowscale_rejects(lib, kw, status):
    assert rowscale(lib, **kw) == status


def test_gemm_rowscale_empty_is_noop(lib):
    assert rowscale(lib, M=0, X=None, Y=None) == OK


@pytest.mark.parametrize("args,status", [
    ((-1, 64, 4, 1e-5, PART_, R2_), SHAPE),
    ((10, 0, 4, 1e-5, PART_, R2_), SHAPE),
    ((10, 64, 0, 1e-5, PART_, R2_), SHAPE),
    ((10, 64, 4, -1.0, PART_, R2_), SHAPE),
    ((10, 64, 4, float("nan"), PART_, R2_), SHAPE),
    ((10, 64, 4, 1e-5, None, R2_), NULL),
    ((10, 64, 4, 1e-5, PART_, None), NULL),
    ((10, 64, 4, 1e-5, PART_ + 2, R2_), ALIGN),
    ((10, 64, 4, 1e-5, PART_, PART_ + 40), ALIAS),
    ((0, 64, 4, 1e-5, None, None), OK),
])
def test_rms_combine_validation(lib, args, status):
    assert lib.coda_rms_combine(*args, None) == status


def test_ref_chain_validation(lib):
    need = lib.coda_ref_chain_workspace_bytes(BF16, 512, 256)

    def call(ws=WS_, ws_bytes=need, **kw):
        a = dict(dt=BF16, M=512, K=256, D=256, N2=512, eps=1e-5, A=A_, W1=W1_, R=R_, g=G_, W2=W2_, H=H_,
                 r=R2_, Y=Y_)
        a.update(kw)
        return lib.coda_ref_chain(a["dt"], a["M"], a["K"], a["D"], a["N2"], a["eps"], a["A"], a["W1"], a["R"],
                                  a["g"], a["W2"], a["H"], a["r"], a["Y"], ws, ws_bytes, None)

    assert call(ws_bytes=need - 1) == WS
    assert call(ws=None) == WS
    assert call(ws=WS_ + 16) == ALIGN
    assert call(g=None) == NULL
    assert call(eps=-1.0) == SHAPE
    assert call(Y=A_) == ALIAS
    assert call(ws=H_ - 1024 * 256) == ALIAS  # workspace overlapping H
    assert call(M=0, A=None) == OK


def swiglu(lib, dt=BF16, M=512, D=256, F=256, X=H_, ldx=None, W2=W2_, ldw2=None, r=R2_, Z=Y_, ldz=None,
           Y=DY_, ldy=None):
    return lib.coda_gemm_rowscale_swiglu(dt, M, D, F, X, ldx or D, W2, ldw2 or 2 * F, r, Z, ldz or F, Y,
                                         ldy or 2 * F, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=4), DTYPE),
    (dict(F=0), SHAPE),
    (dict(F=12), SHAPE),
    (dict(F=264), SHAPE),         # not a multiple of 32
    (dict(D=20), SHAPE),
    (dict(X=None), NULL),
    (dict(W2=None), NULL),
    (dict(Z=None), NULL),
    (dict(ldw2=256), SHAPE),      # ld < 2F
    (dict(ldz=100), SHAPE),       # ld < F
    (dict(ldy=516), ALIGN),       # not a multiple of 8 elements
    (dict(Z=Y_ + 8), ALIGN),
    (dict(r=R2_ + 1), ALIGN),
    (dict(Z=H_), ALIAS),
    (dict(Y=W2_ + 1024), ALIAS),
    (dict(Y=Y_ + 512), ALIAS),    # Z and Y overlapping
    (dict(Z=R2_), ALIAS),
])
def test_gemm_rowscale_swiglu_rejects(lib, kw, status):
    assert swiglu(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


def test_gemm_rowscale_swiglu_empty_is_noop(lib):
    assert swiglu(lib, M=0, X=None, Z=None, Y=None, r=None) == OK


@pytest.mark.parametrize("args,status", [
    ((BF16, 512, 0, DY_, 0, Y_, 0, DA_, 0), SHAPE),
    ((BF16, 512, 100, DY_, 100, Y_, 200, DA_, 200), SHAPE),
    ((7, 512, 256, DY_, 256, Y_, 512, DA_, 512), DTYPE),
    ((BF16, 512, 256, None, 256, Y_, 512, DA_, 512), NULL),
    ((BF16, 512, 256, DY_, 256, None, 512, DA_, 512), NULL),
    ((BF16, 512, 256, DY_, 256, Y_, 512, None, 512), NULL),
    ((BF16, 512, 256, DY_, 256, Y_, 256, DA_, 512), SHAPE),     # ldy < 2F
    ((BF16, 512, 256, DY_, 260, Y_, 512, DA_, 512), ALIGN),
    ((BF16, 512, 256, DY_, 256, Y_, 512, Y_ + 1024, 512), ALIAS),
    ((BF16, 512, 256, DY_, 256, Y_, 512, DY_, 512), ALIAS),
    ((BF16, 0, 256, None, 256, None, 512, None, 512), OK),
])
def test_swiglu_bwd_validation(lib, args, status):
    assert lib.coda_swiglu_bwd(*args, None) == status


def lse_call(lib, dt=BF16, M=512, D=256, V=1000, X=H_, ldx=None, W=W2_, ldw=None, r=R2_, t=DY_, pm=PART_,
             ps=PART_ + (1 << 24), tg=DG_):
    return lib.coda_gemm_rowscale_lse(dt, M, D, V, X, ldx or D, W, ldw or V, r, t, pm, ps, tg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE),
    (dict(V=1001), SHAPE),
    (dict(X=None), NULL),
    (dict(W=None), NULL),
    (dict(t=None), NULL),
    (dict(pm=None), NULL),
    (dict(ps=None), NULL),
    (dict(tg=None), NULL),
    (dict(pm=PART_ + 2), ALIGN),
    (dict(t=DY_ + 1), ALIGN),
    (dict(ldw=996), SHAPE),
    (dict(ps=PART_ + 4096), ALIAS),    # the two statistics arrays overlapping
    (dict(tg=H_), ALIAS),
    (dict(pm=DY_), ALIAS),
])
def test_gemm_rowscale_lse_rejects(lib, kw, status):
    assert lse_call(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((-1, 1000, 16, PART_, R_, DG_, DY_, DA_, DR_), SHAPE),
    ((512, 0, 16, PART_, R_, DG_, DY_, DA_, DR_), SHAPE),
    ((512, 1000, 0, PART_, R_, DG_, DY_, DA_, DR_), SHAPE),
    ((512, 1000, 16, None, R_, DG_, DY_, DA_, DR_), NULL),
    ((512, 1000, 16, PART_, R_, DG_, DY_, None, DR_), NULL),
    ((512, 1000, 16, PART_ + 1, R_, DG_, DY_, DA_, DR_), ALIGN),
    ((512, 1000, 16, PART_, R_, DG_, DY_, PART_ + 64, DR_), ALIAS),
    ((512, 1000, 16, PART_, R_, DG_, DY_, DA_, DA_ + 8), ALIAS),
    ((0, 1000, 16, None, None, None, None, None, None), OK),
])
def test_ce_combine_validation(lib, args, status):
    assert lib.coda_ce_combine(*args, None) == status


def ce_bwd_call(lib, dt=BF16, M=512, D=256, V=1000, X=H_, ldx=None, W=W2_, ldw=None, r=R2_, t=DY_, lse=DG_,
                dl=DG_ + 4096, dY=Y_, lddy=None):
    return lib.coda_gemm_rowscale_ce_bwd(dt, M, D, V, X, ldx or D, W, ldw or V, r, t, lse, dl, dY, lddy or V, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE),
    (dict(V=1001), SHAPE),
    (dict(X=None), NULL),
    (dict(t=None), NULL),
    (dict(lse=None), NULL),
    (dict(dl=None), NULL),
    (dict(dY=None), NULL),
    (dict(lse=DG_ + 2), ALIGN),
    (dict(lddy=1004), ALIGN),
    (dict(dY=DG_ - 64), ALIAS),       # dY over lse
    (dict(dY=W2_ + 512), ALIAS),
    (dict(M=0, X=None, t=None), OK),
])
def test_gemm_rowscale_ce_bwd_rejects(lib, kw, status):
    assert ce_bwd_call(lib, **kw) == status


def test_quantize_validation(lib):
    q = lib.coda_quantize_rows_e4m3
    assert q(512, 264, H_, 264, HG_, 264, PART_, None) == SHAPE            # K not a multiple of 16
    assert q(512, 256, None, 256, HG_, 256, PART_, None) == NULL
    assert q(512, 256, H_, 256, HG_, 256, None, None) == NULL
    assert q(512, 256, H_, 260, HG_, 256, PART_, None) == ALIGN            # ldx not a multiple of 8
    assert q(512, 256, H_, 256, HG_, 264, PART_, None) == ALIGN            # ldx8 not a multiple of 16
    assert q(512, 256, H_, 256, PART_ + 2, 256, PART_, None) == ALIGN
    assert q(512, 256, H_, 256, H_ + 4096, 256, PART_, None) == ALIAS      # codes over X
    assert q(512, 256, H_, 256, HG_, 256, H_ + 64, None) == ALIAS          # scales over X
    assert q(0, 256, None, 256, None, 256, None, None) == OK
    c = lib.coda_quantize_cols_e4m3
    assert c(256, 264, W1_, 264, HG_, 256, PART_, None) == SHAPE            # N not a multiple of 16
    assert c(264, 256, W1_, 256, HG_, 264, PART_, None) == SHAPE            # K not a multiple of 16
    assert c(256, 512, None, 512, HG_, 256, PART_, None) == NULL
    assert c(256, 512, W1_, 512, W1_ + 1024, 256, PART_, None) == ALIAS
    assert c(256, 512, W1_, 512, HG_, 256, PART_ + 1, None) == ALIGN
    rc = lib.coda_quantize_rows_cols_e4m3
    assert rc(520, 256, H_, 256, HG_, 256, PART_, Y_, 520, R2_, None) == SHAPE      # M not a multiple of 16
    assert rc(512, 264, H_, 264, HG_, 264, PART_, Y_, 512, R2_, None) == SHAPE      # N not a multiple of 16
    assert rc(512, 256, None, 256, HG_, 256, PART_, Y_, 512, R2_, None) == NULL
    assert rc(512, 256, H_, 256, HG_, 256, None, Y_, 512, R2_, None) == NULL
    assert rc(512, 256, H_, 256, HG_, 256, PART_, Y_, 520, R2_, None) == ALIGN      # ldxt not a multiple of 16
    assert rc(512, 256, H_, 256, HG_, 256, PART_, Y_, 512, R2_ + 2, None) == ALIGN
    assert rc(512, 256, H_, 256, H_ + 4096, 256, PART_, Y_, 512, R2_, None) == ALIAS  # row codes over X
    assert rc(512, 256, H_, 256, HG_, 256, PART_, HG_ + 256, 512, R2_, None) == ALIAS  # the two code arrays
    assert rc(512, 256, H_, 256, HG_, 256, PART_, Y_, 512, PART_ + 64, None) == ALIAS  # the two scale arrays
    assert rc(0, 256, None, 256, None, 256, None, None, 0, None, None) == OK


def test_quantize_packed_validation(lib):
    q = lib.coda_quantize_rows_e4m3_packed
    assert q(512, 264, H_, 264, HG_, PART_, None) == SHAPE                 # K not a multiple of 16
    assert q(512, 256, None, 256, HG_, PART_, None) == NULL
    assert q(512, 256, H_, 256, HG_, None, None) == NULL
    assert q(512, 256, H_, 260, HG_, PART_, None) == ALIGN                 # ldx not a multiple of 8
    assert q(512, 256, H_, 256, HG_ + 8, PART_, None) == ALIGN
    assert q(512, 256, H_, 256, H_ + 4096, PART_, None) == ALIAS           # codes over X
    assert q(512, 256, H_, 256, HG_, HG_ + 512 * 256 - 64, None) == ALIAS  # scales over the codes
    assert q(0, 256, None, 256, None, None, None) == OK
    rc = lib.coda_quantize_rows_cols_e4m3_packed
    assert rc(520, 256, H_, 256, HG_, PART_, Y_, R2_, None) == SHAPE        # M not a multiple of 16
    assert rc(512, 264, H_, 264, HG_, PART_, Y_, R2_, None) == SHAPE        # N not a multiple of 16
    assert rc(512, 256, H_, 256, HG_, PART_, None, R2_, None) == NULL
    assert rc(512, 256, H_, 256, HG_, PART_, Y_, None, None) == NULL
    assert rc(512, 256, H_, 256, HG_, PART_, Y_ + 4, R2_, None) == ALIGN
    assert rc(512, 256, H_, 256, HG_, PART_, HG_ + 256, R2_, None) == ALIAS  # the two code arrays
    assert rc(512, 256, H_, 256, HG_, PART_, Y_, PART_ + 64, None) == ALIAS  # the two scale arrays
    assert rc(0, 256, None, 256, None, None, None, None, None) == OK


def test_quantize_mx_validation(lib):
    q = lib.coda_quantize_mx_e4m3_packed
    M, N = 512, 256
    assert q(520, N, H_, N, HG_, EX_, Y_, DG_, None) == SHAPE           # M not a multiple of 16
    assert q(M, 264, H_, 264, HG_, EX_, Y_, DG_, None) == SHAPE         # N not a multiple of 16
    assert q(M, 65536 * 256, H_, 65536 * 256, HG_, EX_, None, None, None) == SHAPE  # N past the grid
    assert q(M, N, H_, N, HG_, None, Y_, DG_, None) == NULL             # row codes without exponents
    assert q(M, N, H_, N, HG_, EX_, None, DG_, None) == NULL            # column exponents without codes
    assert q(M, N, H_, N, None, None, None, None, None) == NULL         # no output at all
    assert q(M, N, None, N, HG_, EX_, None, None, None) == NULL
    assert q(M, N, H_, 260, HG_, EX_, None, None, None) == ALIGN        # ldx not a multiple of 8
    assert q(M, N, H_, N, HG_, EX_ + 8, None, None, None) == ALIGN
    assert q(M, N, H_, N, None, None, Y_ + 4, DG_, None) == ALIGN
    assert q(M, N, H_, N, H_ + 4096, EX_, None, None, None) == ALIAS    # codes over X
    assert q(M, N, H_, N, HG_, HG_ + 256, None, None, None) == ALIAS    # exponents over the codes
    assert q(M, N, H_, N, HG_, EX_, HG_ + 4096, DG_, None) == ALIAS     # the two code arrays
    assert q(M, N, H_, N, HG_, EX_, Y_, EX_ + 1024, None) == ALIAS      # the two exponent arrays
    assert q(0, N, None, N, HG_, EX_, None, None, None) == OK           # M = 0: nothing to do
    # the exponent arrays the call fills: 1 KiB per 128 rows and 256 columns
    assert lib.coda_mx_exp_bytes(M, N) == 4096 and lib.coda_mx_exp_bytes(N, M) == 4096


def rope_call(lib, dt=BF16, M=512, D=256, N2=1536, X=H_, ldx=None, W=W2_, ldw=None, r=R2_, pos=DY_, cs=DG_,
              max_pos=2048, nq=512, nk=512, dh=128, Y=Y_, ldy=None):
    return lib.coda_gemm_rowscale_rope(dt, M, D, N2, X, ldx or D, W, ldw or N2, r, pos, cs, max_pos, nq, nk, dh, Y,
                                       ldy or N2, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=5), DTYPE),
    (dict(dh=100), SHAPE),            # not a multiple of 8
    (dict(dh=0), SHAPE),
    (dict(nq=500), SHAPE),            # not whole heads
    (dict(nk=-128), SHAPE),
    (dict(nq=1024, nk=640), SHAPE),   # more rotated columns than the width
    (dict(max_pos=0), SHAPE),
    (dict(pos=None), NULL),
    (dict(cs=None), NULL),
    (dict(Y=None), NULL),
    (dict(pos=DY_ + 2), ALIGN),
    (dict(cs=DG_ + 8), ALIGN),
    (dict(ldy=1540), ALIGN),
    (dict(Y=DG_ + 4096), ALIAS),      # Y over the table
    (dict(Y=DY_), ALIAS),             # Y over the positions
    (dict(Y=H_ + 64), ALIAS),
])
def test_gemm_rowscale_rope_rejects(lib, kw, status):
    assert rope_call(lib, **kw) == status


def test_rope_empty_and_cache_validation(lib):
    assert rope_call(lib, M=0, pos=None, cs=None) == OK
    assert rope_call(lib, M=0, dh=12) == SHAPE
    assert lib.coda_rope_cache(DG_, 2048, 127, 10000.0, None) == SHAPE
    assert lib.coda_rope_cache(DG_, 0, 128, 10000.0, None) == SHAPE
    assert lib.coda_rope_cache(DG_, 2048, 128, 0.0, None) == SHAPE
    assert lib.coda_rope_cache(DG_, 2048, 128, float("inf"), None) == SHAPE
    assert lib.coda_rope_cache(None, 2048, 128, 10000.0, None) == NULL
    assert lib.coda_rope_cache(DG_ + 4, 2048, 128, 10000.0, None) == ALIGN
    assert lib.coda_rope_cache(DG_, 1 << 22, 256, 10000.0, None) == SHAPE   # 4 GiB table


@pytest.mark.parametrize("args,status", [
    ((5, 512, 1536, Y_, 1536, DY_, DG_, 2048, 512, 512, 128, DA_, 1536), DTYPE),
    ((BF16, 512, 1536, Y_, 1536, DY_, DG_, 2048, 512, 512, 96 + 4, DA_, 1536), SHAPE),
    ((BF16, 512, 1536, None, 1536, DY_, DG_, 2048, 512, 512, 128, DA_, 1536), NULL),
    ((BF16, 512, 1536, Y_, 1536, None, DG_, 2048, 512, 512, 128, DA_, 1536), NULL),
    ((BF16, 512, 1536, Y_, 1536, DY_, DG_, 2048, 512, 512, 128, Y_ + 64, 1536), ALIAS),
    ((BF16, 512, 1536, Y_, 1536, DY_, DG_, 2048, 512, 512, 128, DG_, 1536), ALIAS),
    ((BF16, 0, 1536, None, 1536, None, None, 2048, 512, 512, 128, None, 1536), OK),
])
def test_rope_bwd_validation(lib, args, status):
    assert lib.coda_rope_bwd(*args, None) == status


def prms8(lib, M=512, K=256, D=512, A=A_, lda=None, sa=R2_, W=W1_, ldw=None, sw=G_ + 4096, R=R_, ldr=None, g=G_,
           H=H_, ldh=None, Hg=HG_, ldhg=None, ex=EX_, part=PART_):
    return lib.coda_gemm_res_prms_fp8(M, K, D, A, lda or K, sa, W, ldw or K, sw, R, ldr or D, g, H, ldh or D, Hg,
                                      ldhg or D, ex, part, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=8), SHAPE),            # fp8 sizes are multiples of 16
    (dict(D=520), SHAPE),
    (dict(M=-1), SHAPE),
    (dict(A=None), NULL),
    (dict(sa=None), NULL),
    (dict(W=None), NULL),
    (dict(sw=None), NULL),
    (dict(R=None), NULL),
    (dict(g=None), NULL),
    (dict(H=None), NULL),
    (dict(Hg=None), NULL),
    (dict(ex=None), NULL),         # the block exponents are an output of the first GEMM
    (dict(part=None), NULL),
    (dict(ex=EX_ + 4), ALIGN),
    (dict(ex=HG_ + 512 * 512 - 64), ALIAS),   # overlaps Hg8's last row
    (dict(lda=264), ALIGN),        # e4m3 ld must be a multiple of 16 elements
    (dict(ldhg=520), ALIGN),
    (dict(ldr=516), ALIGN),        # bf16 ld a multiple of 8
    (dict(sw=G_ + 4), ALIGN),      # column scales read 16 bytes at a time
    (dict(sa=R2_ + 2), ALIGN),
    (dict(ldw=128), SHAPE),
    (dict(Hg=A_ + 64), ALIAS),
    (dict(H=R_), ALIAS),
    (dict(part=HG_ + 256), ALIAS),
])
def test_gemm_res_prms_fp8_rejects(lib, kw, status):
    assert prms8(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


def rowscale8(lib, M=512, D=256, N2=512, X=HG_, ldx=None, ex=EX_, W=W2_, ldw=None, sw=G_, r=R2_, Y=Y_, ldy=None):
    return lib.coda_gemm_rowscale_fp8(M, D, N2, X, ldx or D, ex, W, ldw or D, sw, r, Y, ldy or N2, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N2=24), SHAPE),
    (dict(X=None), NULL),
    (dict(W=None), NULL),
    (dict(sw=None), NULL),
    (dict(Y=None), NULL),
    (dict(ldx=264), ALIGN),
    (dict(sw=G_ + 8), ALIGN),
    (dict(Y=HG_), ALIAS),
    (dict(Y=G_ - 64), ALIAS),
    (dict(ex=EX_ + 2), ALIGN),
    (dict(Y=EX_ - 64), ALIAS),     # Y's last bytes over the exponents
])
def test_gemm_rowscale_fp8_rejects(lib, kw, status):
    assert rowscale8(lib, **kw) == status


def test_mx_exp_bytes(lib):
    # 1 KiB per 128-row block and group of 4 k-tiles (256 columns)
    assert lib.coda_mx_exp_bytes(300, 512) == 1024 * 3 * 2
    assert lib.coda_mx_exp_bytes(3, 272) == 1024 * 1 * 2
    assert lib.coda_mx_exp_bytes(128, 256) == 1024
    assert lib.coda_mx_exp_bytes(129, 256) == 2048
    assert lib.coda_mx_exp_bytes(1, 16) == 1024
    assert lib.coda_mx_exp_bytes(0, 4096) == 0
    assert lib.coda_mx_exp_bytes(-1, 16) == -1
    assert lib.coda_mx_exp_bytes(4, 0) == -1


def test_fp8_empty_is_noop(lib):
    assert prms8(lib, M=0, A=None, sa=None, R=None, H=None, Hg=None, ex=None, part=None) == OK
    assert rowscale8(lib, M=0, X=None, ex=None, Y=None, r=None) == OK


def test_chain_bwd_workspace_bytes(lib):
    def al(x):
        return (x + 255) // 256 * 256
    # X_n [M, D] (dtype), row partials [T, M], column partials [ceil(M/128), D],
    # c [M], W2^T [N2, D] and W1^T [D, K] (dtype)
    M, K, D, N2 = 16384, 4096, 4096, 28672
    xn = al(M * D * 2)
    srow = al(xn + 64 * M * 4)
    dgcol = al(srow + (M // 128) * D * 4)
    w2t = al(dgcol + M * 4)
    w1t = al(w2t + N2 * D * 2)
    assert lib.coda_chain_bwd_workspace_bytes(BF16, M, K, D, N2) == al(w1t + D * K * 2)
    M, K, D, N2 = 300, 8, 264, 16   # ragged: T = 8, U = 3
    xn = al(M * D * 4)
    srow = al(xn + 8 * M * 4)
    dgcol = al(srow + 3 * D * 4)
    w2t = al(dgcol + M * 4)
    w1t = al(w2t + N2 * D * 4)
    assert lib.coda_chain_bwd_workspace_bytes(F32, M, K, D, N2) == al(w1t + D * K * 4)
    assert lib.coda_chain_bwd_workspace_bytes(7, 16, 8, 8, 8) == 0
    assert lib.coda_chain_bwd_workspace_bytes(BF16, -1, 8, 8, 8) == 0
    assert lib.coda_chain_bwd_workspace_bytes(BF16, 16, 0, 8, 8) == 0


def chain_bwd(lib, ws=WS_, ws_bytes=None, **kw):
    a = dict(dt=BF16, M=512, K=256, D=256, N2=512, dY=DY_, A=A_, W1=W1_, g=G_, W2=W2_, H=H_, r=R2_, dA=DA_,
             dR=DR_, dW1=DW1_, dW2=DW2_, dg=DG_)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.coda_chain_bwd_workspace_bytes(a["dt"] if a["dt"] in (0, 1) else 0, max(a["M"], 0),
                                                      max(a["K"], 1), max(a["D"], 1), max(a["N2"], 1))
    return lib.coda_chain_bwd(a["dt"], a["M"], a["K"], a["D"], a["N2"], a["dY"], a["A"], a["W1"], a["g"],
                              a["W2"], a["H"], a["r"], a["dA"], a["dR"], a["dW1"], a["dW2"], a["dg"], ws,
                              ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), DTYPE),
    (dict(M=-3), SHAPE),
    (dict(K=12), SHAPE),
    (dict(D=0), SHAPE),
    (dict(N2=100), SHAPE),
    (dict(dY=None), NULL),
    (dict(A=None), NULL),
    (dict(W1=None), NULL),
    (dict(g=None), NULL),
    (dict(W2=None), NULL),
    (dict(H=None), NULL),
    (dict(r=None), NULL),
    (dict(dA=None), NULL),
    (dict(dR=None), NULL),
    (dict(dW1=None), NULL),
    (dict(dW2=None), NULL),
    (dict(dg=None), NULL),
    (dict(ws=None), WS),
    (dict(ws_bytes=1024), WS),
    (dict(ws=WS_ + 128), ALIGN),
    (dict(dY=DY_ + 8), ALIGN),
    (dict(r=R2_ + 1), ALIGN),
    (dict(dg=DG_ + 2), ALIGN),
    (dict(dR=H_), ALIAS),            # dH may not overwrite the stored H
    (dict(dA=A_ + 512), ALIAS),
    (dict(dW2=W2_), ALIAS),
    (dict(dg=R2_), ALIAS),
    (dict(dW1=DR_ + 4096), ALIAS),   # two outputs overlapping
    (dict(ws=DY_), ALIAS),           # workspace overlapping an input
    (dict(ws=DW2_ - 256), ALIAS),    # workspace overlapping an output
    (dict(M=16384, N2=65536), SHAPE),  # dY spans more than 2 GiB
])
def test_chain_bwd_rejects(lib, kw, status):
    assert chain_bwd(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


def chain_bwd_noalloc(lib, **kw):
    a = dict(dt=BF16, M=512, K=256, D=256, N2=512, dY=DY_, A=A_, W1=W1_, g=G_, W2=W2_, H=H_, r=R2_, dA=DA_,
             dR=DR_, dW1=DW1_, dW2=DW2_, dg=DG_)
    a.update(kw)
    return lib.coda_chain_bwd_noalloc(a["dt"], a["M"], a["K"], a["D"], a["N2"], a["dY"], a["A"], a["W1"], a["g"],
                                      a["W2"], a["H"], a["r"], a["dA"], a["dR"], a["dW1"], a["dW2"], a["dg"], None)


def _noalloc_need(M, D, es):
    al = lambda x: (x + 255) // 256 * 256
    T, U = 4 * ((D + 255) // 256), (M + 127) // 128
    return al(al(al(al(M * D * es) + T * M * 4) + U * D * 4) + M * 4)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), DTYPE),
    (dict(K=12), SHAPE),
    (dict(dY=None), NULL),
    (dict(dg=None), NULL),
    (dict(r=R2_ + 1), ALIGN),
    (dict(dR=H_), ALIAS),
    (dict(dW1=DR_ + 4096), ALIAS),
    (dict(M=7936, D=4096, K=256, N2=512), WS),    # X_n and the partial sums just over the 64 MiB scratch
    (dict(M=16384, D=4096, K=4096, N2=28672), WS),  # the 7B backward needs a workspace
])
def test_chain_bwd_noalloc_rejects(lib, kw, status):
    # validation happens before anything touches a device (so these run
    # without a GPU); shapes whose scratch exceeds the static array fail
    assert chain_bwd_noalloc(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


def test_chain_bwd_noalloc_limit():
    # the header's limit and the scratch the two rejected shapes need
    assert _noalloc_need(7680, 4096, 2) <= 64 << 20 < _noalloc_need(7936, 4096, 2)
    hdr = open(HEADER).read()
    assert "#define CODA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in hdr


def test_chain_bwd_empty_still_checks_weights(lib):
    # with M = 0 the M-row arguments may be NULL, the weight gradients may not
    none = dict(dY=None, A=None, H=None, r=None, dA=None, dR=None)
    assert chain_bwd(lib, M=0, dW1=None, **none) == NULL
    assert chain_bwd(lib, M=0, dg=None, **none) == NULL
    assert chain_bwd(lib, M=0, dW2=W2_, **none) == ALIAS


def test_index_maps_host_check(tmp_path):
    exe = tmp_path / "tile_map_check"
    src = os.path.join(ROOT, "tests", "host", "tile_map_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-o", str(exe), src], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr


def test_package_without_library_fails_loudly(tmp_path):
    # the binding has no fallback: a copy of the package without libcoda.so
    # must refuse to import
    import shutil
    import sys as _sys
    src = os.path.join(ROOT, "transformer_gemm_epilogue_gemm1_amd")
    dst = tmp_path / "transformer_gemm_epilogue_gemm1_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__", "csrc"))
    assert not any(p.suffix == ".so" for p in dst.iterdir())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import transformer_gemm_epilogue_gemm1_amd\nexcept ImportError as e:\n"
            "    print('ImportError:', e); sys.exit(3)\nsys.exit(0)\n") % str(tmp_path)
    out = subprocess.run([_sys.executable, "-c", code], capture_output=True, text=True, cwd=str(tmp_path))
    assert out.returncode == 3, out.stdout + out.stderr
    assert "libcoda.so not built" in out.stdout


def test_chain_bwd_fp8_validation(lib):
    M, K, D, N2 = 512, 256, 512, 768
    need = lib.coda_chain_bwd_fp8_workspace_bytes(M, K, D, N2)
    assert need > lib.coda_chain_bwd_workspace_bytes(BF16, M, K, D, N2)   # plus the e4m3 operands
    assert lib.coda_chain_bwd_fp8_workspace_bytes(-1, K, D, N2) == 0

    def call(M=M, K=K, D=D, N2=N2, dY=DY_, ws=WS_, ws_bytes=None, r=R2_, dW2=DW2_):
        return lib.coda_chain_bwd_fp8(M, K, D, N2, dY, A_, W1_, G_, W2_, H_, r, DA_, DR_, DW1_, dW2, DG_, ws,
                                      need if ws_bytes is None else ws_bytes, None)
    assert call(M=520) == SHAPE            # M not a multiple of 16
    assert call(D=520) == SHAPE
    assert call(dY=None) == NULL
    assert call(r=None) == NULL
    assert call(ws_bytes=need - 1) == WS
    assert call(ws=WS_ + 8) == ALIGN
    assert call(dW2=W2_ + 64) == ALIAS


def test_ceiling_library_exports_and_rejects():
    """The benchmark's matrix-core throughput library exports its two calls
    and turns bad arguments into -1 before any launch."""
    import ctypes

    from transformer_gemm_epilogue_gemm1_amd.build import CEILING_LIB_PATH

    lib = ctypes.CDLL(CEILING_LIB_PATH)
    for kind in ("bf16", "fp8"):
        fn = getattr(lib, f"coda_ceiling_{kind}")
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                       ctypes.c_void_p]
        fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is rejected first
        assert fn(None, 1 << 20, 2048, 1, 0, None) == -1
        assert fn(fake, 2048 * 512 - 1, 2048, 1, 0, None) == -1
        assert fn(fake, 2048 * 512, 0, 1, 0, None) == -1
        assert fn(fake, 2048 * 512, 2048, 0, 0, None) == -1


# ---- the forward pair with Hg tile-packed ----
def test_packed_bytes(lib):
    assert lib.coda_packed_bytes(300, 512) == 304 * 512 * 2
    assert lib.coda_packed_bytes(16, 8) == 16 * 8 * 2
    assert lib.coda_packed_bytes(0, 8) == 0
    assert lib.coda_packed_bytes(1, 12) == -1
    assert lib.coda_packed_bytes(-1, 8) == -1
    assert lib.coda_packed_bytes(1, 0) == -1


def prms_packed(lib, M=300, K=256, D=512, A=A_, lda=256, W1=W1_, ldw1=512, R=R_, ldr=512, g=G_, H=H_, ldh=512,
                Hgp=HG_, part=PART_):
    return lib.coda_gemm_res_prms_packed(M, K, D, A, lda, W1, ldw1, R, ldr, g, H, ldh, Hgp, part, None)


def rowscale_packed(lib, M=300, D=512, N2=768, Xp=HG_, W2=W2_, ldw2=768, r=R2_, Y=Y_, ldy=768):
    return lib.coda_gemm_rowscale_packed(M, D, N2, Xp, W2, ldw2, r, Y, ldy, None)


@pytest.mark.parametrize("kw,status", [
    (dict(D=500), SHAPE),
    (dict(g=None), NULL),
    (dict(Hgp=None), NULL),
    (dict(Hgp=HG_ + 8), ALIGN),
    (dict(part=PART_ + 2), ALIGN),
    (dict(ldh=256), SHAPE),
    (dict(Hgp=H_ + 64), ALIAS),   # overlaps H
    (dict(Hgp=R_), ALIAS),
])
def test_gemm_res_prms_packed_rejects(lib, kw, status):
    assert prms_packed(lib, **kw) == status
    assert lib.coda_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(N2=12), SHAPE),
    (dict(Xp=None), NULL),
    (dict(Xp=HG_ + 4), ALIGN),
    (dict(ldy=256), SHAPE),
    (dict(Y=HG_ + 1024), ALIAS),
    (dict(r=R2_ + 2), ALIGN),
])
def test_gemm_rowscale_packed_rejects(lib, kw, status):
    assert rowscale_packed(lib, **kw) == status


def test_packed_pair_empty_is_noop(lib):
    assert prms_packed(lib, M=0, A=None, R=None, H=None, Hgp=None, part=None) == OK
    assert rowscale_packed(lib, M=0, Xp=None, Y=None) == OK


def test_fp8_packed_validation(lib):
    assert lib.coda_packed_bytes_e4m3(300, 512) == 304 * 512
    assert lib.coda_packed_bytes_e4m3(1, 8) == -1
    # quantiser: N not a multiple of 16, NULL output, misaligned output, output overlapping W
    assert lib.coda_quantize_cols_e4m3_packed(256, 24, W2_, 24, WS_, R2_, None) == SHAPE
    assert lib.coda_quantize_cols_e4m3_packed(256, 512, W2_, 512, None, R2_, None) == NULL
    assert lib.coda_quantize_cols_e4m3_packed(256, 512, W2_, 512, WS_ + 8, R2_, None) == ALIGN
    assert lib.coda_quantize_cols_e4m3_packed(256, 512, W2_, 512, W2_ + 64, R2_, None) == ALIAS
    # first GEMM: Hg8 overlapping H
    assert lib.coda_gemm_res_prms_fp8_packed(300, 256, 512, A_, 256, R2_, W1_, 256, DG_, R_, 512, G_, H_, 512,
                                             H_ + 64, EX_, PART_, None) == ALIAS
    # first GEMM: exponents missing, or overlapping the packed Hg8
    assert lib.coda_gemm_res_prms_fp8_packed(300, 256, 512, A_, 256, R2_, W1_, 256, DG_, R_, 512, G_, H_, 512,
                                             HG_, None, PART_, None) == NULL
    assert lib.coda_gemm_res_prms_fp8_packed(300, 256, 512, A_, 256, R2_, W1_, 256, DG_, R_, 512, G_, H_, 512,
                                             HG_, HG_ + 1024, PART_, None) == ALIAS
    # second GEMM: D not a multiple of 16, NULL operand, Y overlapping X or the exponents
    assert lib.coda_gemm_rowscale_fp8_packed(300, 264, 512, HG_, EX_, W2_, DG_, R2_, Y_, 512, None) == SHAPE
    assert lib.coda_gemm_rowscale_fp8_packed(300, 256, 512, None, EX_, W2_, DG_, R2_, Y_, 512, None) == NULL
    assert lib.coda_gemm_rowscale_fp8_packed(300, 256, 512, HG_, EX_, W2_, DG_, R2_, HG_ + 16, 512, None) == ALIAS
    assert lib.coda_gemm_rowscale_fp8_packed(300, 256, 512, HG_, EX_, W2_, DG_, R2_, EX_ + 16, 512, None) == ALIAS
    assert lib.coda_gemm_rowscale_fp8_packed(300, 256, 512, HG_, EX_ + 8, W2_, DG_, R2_, Y_, 512, None) == ALIGN
    assert lib.coda_gemm_rowscale_fp8_packed(0, 256, 512, None, None, None, None, None, None, 512, None) == OK


def test_fp8_all_packed_first_gemm_validation(lib):
    def call(M=300, K=256, D=512, A8p=A_, sa=R2_, W1t8p=W1_, sw1=DG_, R=R_, ldr=512, H=H_, Hg8p=HG_, ex=EX_,
             part=PART_):
        return lib.coda_gemm_res_prms_fp8_all_packed(M, K, D, A8p, sa, W1t8p, sw1, R, ldr, G_, H, 512, Hg8p, ex,
                                                     part, None)
    assert call(K=264) == SHAPE            # K not a multiple of 16
    assert call(D=520) == SHAPE
    assert call(ldr=256) == SHAPE          # R's leading dimension below D
    assert call(A8p=None) == NULL
    assert call(W1t8p=None) == NULL
    assert call(ex=None) == NULL
    assert call(A8p=A_ + 8) == ALIGN       # packed codes 16-byte aligned
    assert call(sw1=DG_ + 4) == ALIGN
    assert call(Hg8p=A_ + 64) == ALIAS     # output inside the packed A8p
    assert call(H=W1_ + 1024) == ALIAS     # output inside the packed W1t8p
    assert call(M=0, A8p=None, W1t8p=None, R=None, H=None, Hg8p=None, ex=None, part=None) == OK


def test_lse_ce_rope_packed_validation(lib):
    # LM head with the cross-entropy statistics: M=300, D=512, V=1000
    lse = lambda **k: lib.coda_gemm_rowscale_lse_packed(
        k.get("M", 300), k.get("D", 512), k.get("V", 1000), k.get("Xp", HG_), W2_, 1000, R2_,
        k.get("t", DY_), k.get("pmax", DA_), DR_, DW1_, None)
    assert lse(V=1001) == SHAPE
    assert lse(Xp=None) == NULL
    assert lse(t=None) == NULL
    assert lse(Xp=HG_ + 4) == ALIGN
    assert lse(pmax=HG_ + 256) == ALIAS          # statistics written over the packed Hg
    assert lse(M=0, Xp=None, t=None, pmax=None) == OK
    # its backward
    ce = lambda **k: lib.coda_gemm_rowscale_ce_bwd_packed(
        300, k.get("D", 512), 1000, k.get("Xp", HG_), W2_, 1000, R2_, DY_, DA_, DR_, k.get("dY", Y_),
        k.get("lddy", 1000), None)
    assert ce(D=12) == SHAPE
    assert ce(Xp=None) == NULL
    assert ce(lddy=999) == SHAPE
    assert ce(dY=HG_ + 1024) == ALIAS
    # QKV projection with RoPE: N2=1040, n_q=512, n_k=256, d_head=64, max_pos=4096
    rope = lambda **k: lib.coda_gemm_rowscale_rope_packed(
        300, 384, 1040, k.get("Xp", HG_), W2_, 1040, R2_, DY_, k.get("cs", DA_), 4096, k.get("nq", 512), 256, 64,
        k.get("Y", Y_), 1040, None)
    assert rope(nq=500) == SHAPE
    assert rope(Xp=None) == NULL
    assert rope(cs=None) == NULL
    assert rope(Xp=HG_ + 8) == ALIGN
    assert rope(Y=HG_ + 512) == ALIAS


@pytest.mark.parametrize("dim", ["K", "D", "N2"])
@pytest.mark.parametrize("dt", [BF16, F32])
def test_sizes_narrowed_to_multiples_of_8(lib, dim, dt):
    # The boundary takes K, D and N2 in multiples of 8 only (the kernels move
    # 16-byte pieces of 8 bf16 along every one of them, the fp32 path keeps
    # the same rule); any other size is refused with CODA_ERR_SHAPE before
    # anything is enqueued, by the forward pair, the reference chain and the
    # backward alike, and the message names the size.
    base = dict(M=512, K=256, D=256, N2=512)
    bad = dict(base, **{dim: base[dim] + 4})
    calls = []
    if dim in ("K", "D"):
        calls.append(lambda: prms(lib, dt=dt, M=bad["M"], K=bad["K"], D=bad["D"], lda=bad["K"] + 4,
                                  ldw1=bad["D"] + 4, ldr=bad["D"] + 4, ldh=bad["D"] + 4, ldhg=bad["D"] + 4))
    if dim in ("D", "N2"):
        calls.append(lambda: rowscale(lib, dt=dt, M=bad["M"], D=bad["D"], N2=bad["N2"], ldx=bad["D"] + 4,
                                      ldw2=bad["N2"] + 4, ldy=bad["N2"] + 4))
    calls.append(lambda: chain_bwd(lib, dt=dt, ws_bytes=1 << 40, **bad))
    for call in calls:
        assert call() == SHAPE
        assert f"{dim} = {bad[dim]} is not a multiple of 8" in lib.coda_last_error().decode()
    # the same call at the multiple of 8 just below gets past the size check
    assert chain_bwd(lib, dt=dt, ws=None, **dict(base, **{dim: base[dim] - 8})) == WS
