"""Helpers shared by the GPU tests: device copies of host inputs and error metrics."""
import numpy as np
import torch

import coda_inputs as ci


def dev(h: "ci.HostTensor", device="cuda") -> torch.Tensor:
    if h.dtype == "bf16":
        return torch.from_numpy(h.bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(h.bits).to(device)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy().view(np.uint32)


def max_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref| over the whole tensor."""
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / np.max(np.abs(ref)))


def tolerance(dtype: str) -> float:
    return 1e-2 if dtype == "bf16" else 1e-5


def round_to(dtype: str, x: np.ndarray) -> np.ndarray:
    """Host rounding of float32 values to the storage dtype (RNE), as float32."""
    x = np.asarray(x, dtype=np.float32)
    return ci.bf16_bits_to_f32(ci.bf16_bits(x)) if dtype == "bf16" else x


def whole_max_rel(oracle_rows, got, M: int, block: int = 2048, check=None):
    """max|got - ref| / max|ref| over EVERY row of each tensor in `got`.

    The oracle runs on row blocks (exact: no step of the chain mixes rows),
    so the full-size tensors are compared without holding them in float64.
    oracle_rows(rows) -> dict of float64 arrays for those rows; got: name ->
    device tensor with M rows first; check(rows, ref, host) runs extra
    per-block assertions."""
    num = {k: 0.0 for k in got}
    den = {k: 0.0 for k in got}
    for s in range(0, M, block):
        rows = np.arange(s, min(M, s + block))
        ref = oracle_rows(rows)
        host = {k: t[s:s + len(rows)].float().cpu().numpy().astype(np.float64) for k, t in got.items()}
        for k in got:
            num[k] = max(num[k], float(np.max(np.abs(host[k] - ref[k]))))
            den[k] = max(den[k], float(np.max(np.abs(ref[k]))))
        if check is not None:
            check(rows, ref, host)
    return {k: num[k] / den[k] for k in got}
