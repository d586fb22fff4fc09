"""The benchmark's matrix-core throughput kernels (libcoda_ceiling.so): a small
launch completes, fills every output with a finite sum, and repeats bit for
bit with the same seed."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu


def _fn(kind):
    from transformer_gemm_epilogue_gemm1_amd.build import CEILING_LIB_PATH

    lib = ctypes.CDLL(CEILING_LIB_PATH)
    fn = getattr(lib, f"coda_ceiling_{kind}")
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, ctypes.c_void_p]
    return fn


@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_ceiling_kernel_small_launch(kind):
    import torch

    fn = _fn(kind)
    grid = 4
    s = torch.cuda.current_stream()
    outs = []
    for _ in range(2):
        out = torch.full((grid * 512,), float("nan"), device="cuda", dtype=torch.float32)
        assert fn(out.data_ptr(), out.numel(), grid, 10, 7, s.cuda_stream) == 0
        torch.cuda.synchronize()
        outs.append(out)
    assert bool(torch.isfinite(outs[0]).all())
    assert torch.equal(outs[0], outs[1])
    assert float(outs[0].abs().max()) > 0
