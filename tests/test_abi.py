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
A_, W1_, R_, G_, H_, HG_, PART_, W2_, Y_, R2_, WS_ = (P + i * (1 << 36) for i in range(11))


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


def test_index_maps_host_check(tmp_path):
    exe = tmp_path / "tile_map_check"
    src = os.path.join(ROOT, "tests", "host", "tile_map_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-o", str(exe), src], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr
