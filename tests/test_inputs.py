"""Checks of the seeded input generator (host only)."""
import numpy as np
import torch

from gdn2_inputs import make_config_inputs, make_decode_inputs, make_inputs, round_to_bf16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0], np.float32)])
    x = x.astype(np.float32)
    ours = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_distributions_and_exactness():
    x = make_inputs(2, 64, 3, 16, 8, "bf16", seed=5, reset_frac=0.1, s0_std=0.02)
    for n in ("q", "k", "v", "g", "b", "w"):
        assert x[n].dtype == np.float32
        assert np.array_equal(round_to_bf16(x[n]), x[n]), n
    assert x["q"].shape == (2, 64, 3, 16) and x["v"].shape == (2, 64, 3, 8)
    assert np.all(x["g"] <= 0) and np.any(x["g"] == -5.0)
    assert np.all((x["b"] > 0) & (x["b"] < 1)) and np.all((x["w"] > 0) & (x["w"] < 1))
    nrm = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert np.allclose(nrm, 1.0, atol=2e-2)
    assert x["s0"].shape == (2, 3, 16, 8) and abs(float(x["s0"].std()) - 0.02) < 0.005
    reset_rows = np.all(x["g"] == -5.0, axis=-1)
    assert 0.03 < reset_rows.mean() < 0.2


def test_seeded_and_varlen():
    a = make_inputs(1, 32, 2, 8, 8, "fp32", seed=3)
    b = make_inputs(1, 32, 2, 8, 8, "fp32", seed=3)
    assert all(np.array_equal(a[n], b[n]) for n in "qkvgbw")
    v = make_config_inputs("varlen_bf16", N=4, len_lo=3, len_hi=9, H=2, dk=8, dv=8)
    cu = v["cu_seqlens"]
    assert cu.dtype == np.int32 and cu[0] == 0 and len(cu) == 5
    assert v["q"].shape[1] == cu[-1] and v["s0"].shape == (4, 2, 8, 8)
    d = make_decode_inputs(3, 2, 8, 4, steps=5, seed=1)
    assert d["q"].shape == (5, 3, 2, 8) and d["w"].shape == (5, 3, 2, 4)
