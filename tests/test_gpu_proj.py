"""GPU parity of csa_grouped_out_proj against the fp64 oracle: fp32 and bf16
with a ragged token count (several 128-row tiles plus a tail), a decode-size
batch, and sampled rows of the 32K-token prefill (64 heads of 128 in 8 groups
projected to 1024 each)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, dev, f64
from sparse_attention_17_amd import ops
from synth import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T,H,d,G,dg", [(300, 8, 64, 2, 256), (8, 64, 128, 8, 1024), (129, 4, 128, 1, 128)])
def test_all_rows(dtype, T, H, d, G, dg):
    o, w = inputs.proj_inputs(70, T, H, d, G, dg, dtype)
    y = ops.grouped_out_proj(o.to(dev()), w.to(dev()))
    torch.cuda.synchronize()
    assert y.shape == (T, G * dg)
    assert_close(y.cpu(), oracle.proj.grouped_out_proj(f64(o), f64(w)), dtype, f"proj {T}x{H}x{d}/{G}")


def test_prefill_32k_sampled_rows():
    T, H, d, G, dg = 32768, 64, 128, 8, 1024
    o, w = inputs.proj_inputs(71, T, H, d, G, dg, "bf16")
    y = ops.grouped_out_proj(o.to(dev()), w.to(dev())).cpu()
    rows = np.random.default_rng(3).choice(T, 48, replace=False)
    rows = np.concatenate([rows, [0, 127, 128, T - 1]])
    ref = oracle.proj.grouped_out_proj(f64(o[rows]), f64(w))
    assert_close(y[rows], ref, "bf16", "proj 32k sampled")
    assert torch.isfinite(y.float()).all()


def test_zero_tokens():
    o, w = inputs.proj_inputs(70, 0, 8, 64, 2, 128, "bf16")
    assert ops.grouped_out_proj(o.to(dev()), w.to(dev())).shape == (0, 256)
