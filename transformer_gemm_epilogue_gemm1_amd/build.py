"""Builds libcoda.so (HIP, gfx950 only) next to this file with hipcc, and
libcoda_ceiling.so, the benchmark's matrix-core throughput kernel."""
from __future__ import annotations

import os
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libcoda.so")
SOURCES = ["coda.hip"]
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libcoda_ceiling.so")
CEILING_SOURCES = ["mfma_ceiling.hip"]
HEADERS = ["gemm.hpp", "gemm_fp8.hpp", "epilogues.hpp", "epilogues_fp8.hpp", "epilogues_rope.hpp",
           "epilogues_ce.hpp", "quantize_fp8.hpp", "rowops.hpp", "tile_map.hpp"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(sources, out_path, verbose):
    fd, tmp = tempfile.mkstemp(prefix=os.path.basename(out_path)[:-len(".so")] + ".", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [hipcc()] + HIP_FLAGS + ["-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{res.stderr}")
        if verbose:
            print(" ".join(cmd))
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)


def build(verbose: bool = False) -> str:
    """Compile every HIP source: libcoda.so and libcoda_ceiling.so (always recompiles)."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(CEILING_SOURCES, CEILING_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
