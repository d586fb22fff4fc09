"""The library's calls can be captured in a HIP graph and replayed.

Every entry point only enqueues kernels on the caller's stream: no
allocation, no host synchronisation, no memset (buffers that must start at
zero are cleared by fill kernels).  A training step (fused forward and
backward, bf16; and the fp8 step on a bf16 activation) is captured once with
torch.cuda.graph; each replay, with the inputs rewritten in place in
between and eager steps run between the replays, must reproduce the bits of
an eager step on the same inputs.  The eager step itself is checked against
the oracle by the other GPU tests.
"""
import sys

import numpy as np
import pytest
import torch

import coda_inputs as ci
import transformer_gemm_epilogue_gemm1_amd as coda
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.nodeid}", file=sys.__stderr__, flush=True)
    yield
    torch.cuda.synchronize()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _same(a, b):
    return torch.equal(_bits(a), _bits(b))


def _capture_and_compare(step, inputs, refill):
    """step() -> tuple of tensors on the current inputs; refill(i) rewrites
    the inputs in place for round i."""
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for rnd in range(3):
        refill(rnd)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = [o.clone() for o in outs]
        eager = step()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(replayed, eager)):
            assert _same(a, b), f"round {rnd}: output {i} of the replay differs from the eager step"
    return outs


def test_bf16_training_step_graph():
    wl = ci.custom_workload(528, 512, 384, 1040, wl_id=601)
    x = ci.make_inputs(wl, seed=21, with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    gen = torch.Generator(device="cuda")

    def step():
        H, Hg, r, Y, P = coda.fused_forward(d["A"], d["W1"], d["R"], d["g"], d["W2"], wl.eps)
        return (H, Hg, r, Y) + tuple(coda.fused_backward(d["dY"], d["A"], d["W1"], d["g"], d["W2"], H, r))

    def refill(rnd):
        gen.manual_seed(100 + rnd)
        d["A"].copy_(torch.randn(d["A"].shape, device="cuda", generator=gen).to(d["A"].dtype))
        d["dY"].copy_(torch.randn(d["dY"].shape, device="cuda", generator=gen).to(d["dY"].dtype))

    _capture_and_compare(step, d, refill)


def test_fp8_training_step_graph():
    wl = ci.custom_workload(528, 512, 384, 1040, wl_id=602)
    x = ci.make_inputs(wl, seed=22, with_dy=True)
    d = {k: dev(v) for k, v in x.items()}
    gen = torch.Generator(device="cuda")

    def step():
        Wt8, sw1 = coda.quantize_weight_e4m3(d["W1"])
        W2t8, sw2 = coda.quantize_weight_e4m3(d["W2"])
        H, Hg8, E, r, Y, P, A8, sa = coda.fused_forward_fp8_from_bf16(d["A"], Wt8, sw1, d["R"], d["g"], W2t8, sw2,
                                                                      wl.eps)
        grads = coda.fused_backward_fp8(d["dY"], d["A"], d["W1"], d["g"], d["W2"], H, r)
        return (H, Hg8, E, r, Y, A8, sa) + tuple(grads)

    def refill(rnd):
        gen.manual_seed(200 + rnd)
        d["A"].copy_(torch.randn(d["A"].shape, device="cuda", generator=gen).to(d["A"].dtype))
        d["dY"].copy_(torch.randn(d["dY"].shape, device="cuda", generator=gen).to(d["dY"].dtype))
        d["W2"].mul_(0.5 + rnd)

    _capture_and_compare(step, d, refill)
