"""The seeded input generators: determinism, rounding, value recipe (CPU only)."""
import numpy as np
import torch

import coda_inputs as ci


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.0e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ci.bf16_bits(x), ref)
    back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ci.bf16_bits_to_f32(ref), back)


def test_deterministic_and_distinct():
    wl = ci.custom_workload(64, 32, 48, 80)
    a = ci.make_inputs(wl, seed=3, with_dy=True)
    b = ci.make_inputs(wl, seed=3, with_dy=True)
    c = ci.make_inputs(wl, seed=4)
    for k in a:
        np.testing.assert_array_equal(a[k].bits, b[k].bits)
    assert not np.array_equal(a["A"].bits, c["A"].bits)
    assert not np.array_equal(a["A"].f32[:, :32], a["R"].f32[:, :32])


def test_value_recipe():
    wl = ci.custom_workload(512, 256, 384, 640, dtype="f32")
    x = ci.make_inputs(wl, seed=0, with_dy=True)
    assert x["A"].shape == (512, 256) and x["R"].shape == (512, 384)
    assert x["W1"].shape == (256, 384) and x["W2"].shape == (384, 640) and x["g"].shape == (384,)
    assert x["dY"].shape == (512, 640)
    assert abs(x["A"].f32.std() - 1.0) < 0.01 and abs(x["R"].f32.mean()) < 0.01
    assert abs(x["W1"].f32.var() * 256 - 1.0) < 0.02
    assert abs(x["W2"].f32.var() * 384 - 1.0) < 0.02
    assert abs(x["g"].f32.mean() - 1.0) < 0.02 and abs(x["g"].f32.std() - 0.1) < 0.02


def test_named_workloads():
    w = ci.WORKLOADS["7b-bf16"]
    assert (w.M, w.K, w.D, w.N2, w.dtype) == (16384, 4096, 4096, 28672, "bf16")
    assert abs(w.fwd_flops - 4.398e12) < 1e10
    assert ci.WORKLOADS["70b-bf16"].N2 == 57344 and ci.WORKLOADS["1b-bf16"].D == 2048
    t = ci.WORKLOADS["tiny-fp32"]
    assert (t.M, t.K, t.D, t.N2, t.eps, t.dtype) == (256, 256, 256, 512, 1e-6, "f32")
