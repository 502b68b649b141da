"""The seeded generator is deterministic, shaped as the workloads state, and
rounds to the storage dtype with round-to-nearest-even."""
import numpy as np
import torch

from synth import configs, inputs


def test_deterministic_and_shapes_tiny():
    w = configs.TINY
    a, b = inputs.make_inputs(w), inputs.make_inputs(w)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    assert a["k"].shape == (1, 1024, 64) and a["k"].dtype == torch.float32
    assert a["ki"].shape == (1, 1024, 32)
    assert a["q"].shape == (1, 1024, 4, 64) and a["qi"].shape == (1, 1024, 2, 32)
    assert a["w"].shape == (1, 1024, 2)
    np.testing.assert_allclose(a["w"].sum(-1).numpy(), 1.0, rtol=1e-6)
    assert a["sink"].shape == (4,) and a["q_hca"].shape == (1, 1024, 4, 64)


def test_scaling_by_last_dim():
    x = inputs.normal(99, "q", (4096, 128))
    assert abs(float(x.std()) - 128 ** -0.5) < 2e-3


def test_bf16_is_rne():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=torch.float32)
    y = inputs.to_dtype(x, "bf16").float()
    assert y.tolist() == [1.0, 1.0 + 2 ** -6]


def test_decode_shapes_fp8_fp4():
    w = configs.HYBRID_1M_FP8.with_(ctx=4096, B=2)
    a = inputs.make_inputs(w)
    assert a["kic"].dtype == torch.uint8 and a["kic"].shape == (2, 1024, 64)
    assert a["kic_scale"].shape == (2, 1024) and a["qi_scale"].shape == (2, 1, 4)
    assert a["kc_hca"].shape == (2, 32, 128) and a["kw"].shape == (2, 128, 128)
    b = inputs.make_inputs(w.with_(qk_dtype="fp4"))
    assert b["kic"].shape == (2, 1024, 32) and b["kic_scale"].shape == (2, 1024, 2)
    assert b["qi"].shape == (2, 1, 4, 32) and b["qi_scale"].shape == (2, 1, 4, 2)


def test_peaky_scales_queries_and_sinks():
    w = configs.TINY
    a, p = inputs.make_inputs(w), inputs.make_inputs(w, peaky=True)
    assert torch.allclose(p["q"], a["q"] * 256) and torch.allclose(p["sink"], a["sink"] * 4)
