"""Pins for oracle.formats: the OCP format definitions (golden fixture),
torch's own float8_e4m3fn decoder, and encode/decode round trips."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats
from synth import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ocp_fp8_fp4_values.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        fmt, code, val = line.split()
        rows.append((fmt, int(code, 16), float(val)))
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1", "e8m0"])
def test_golden_values(fmt):
    dec = {"e4m3": formats.e4m3_to_f64, "e2m1": formats.e2m1_to_f64,
           "e8m0": formats.e8m0_to_f64}[fmt]
    rows = [r for r in _golden() if r[0] == fmt]
    assert rows
    for _, code, val in rows:
        got = float(dec(np.array([code], dtype=np.uint8))[0])
        assert _same(got, val), (fmt, hex(code), got, val)


def test_e4m3_all_codes_match_torch_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_to_f64(codes.numpy())
    for c in range(256):
        assert _same(float(got[c]), float(ref[c])), (hex(c), got[c], ref[c])


def test_e4m3_monotone_over_positive_codes():
    v = formats.e4m3_to_f64(np.arange(0, 127, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_unpack_low_nibble_first():
    p = np.array([[0x21, 0xF0]], dtype=np.uint8)
    assert formats.unpack_fp4(p).tolist() == [[1, 2, 0, 15]]


def test_fp8_row_round_trip_within_half_ulp():
    x = torch.from_numpy(np.random.default_rng(0).standard_normal((64, 64)).astype(np.float32))
    codes, scale = quant.quant_fp8_rows(x)
    deq = formats.dequant_fp8_rows(codes.numpy(), scale.numpy())
    y = x.double().numpy() / scale.double().numpy()[:, None]
    err = np.abs(deq / scale.double().numpy()[:, None] - y)
    # e4m3 has 3 mantissa bits: half-ulp <= 2^-4 relative for normals, 2^-10 abs below 2^-6
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) + 1e-12
    assert np.all(err <= bound)
    # the row maximum maps to the largest code (amax/scale == 448 up to fp32 rounding)
    assert np.allclose(np.abs(deq).max(axis=1), np.abs(x.double().numpy()).max(axis=1), rtol=2e-7)


def test_fp4_block_round_trip_and_scales():
    x = torch.from_numpy(np.random.default_rng(1).standard_normal((16, 64)).astype(np.float32))
    packed, sc = quant.quant_fp4_blocks(x)
    assert packed.shape == (16, 32) and sc.shape == (16, 2)
    deq = formats.dequant_fp4_blocks(packed.numpy(), sc.numpy())
    xs = x.double().numpy().reshape(16, 2, 32)
    amax = np.abs(xs).max(axis=-1)
    scale = formats.e8m0_to_f64(sc.numpy())
    # MX convention: amax / scale lies in [4, 8)
    assert np.all((amax / scale >= 4) & (amax / scale < 8))
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    y = np.abs(xs / scale[..., None])
    nearest = np.abs(y[..., None] - grid).min(axis=-1)
    got = np.abs(deq.reshape(16, 2, 32) / scale[..., None])
    # decoded magnitude is a nearest grid point (saturating at 6)
    sat = y > 6
    assert np.all(np.isclose(np.abs(got - y), nearest) | (sat & (got == 6)))


def test_fp4_ties_go_to_even_code():
    # element values on exact midpoints after scaling by 1 (amax 6 -> scale 2^0... use amax=4 -> 2^0)
    vals = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] + [0.0] * 24, dtype=np.float32)
    packed, sc = quant.quant_fp4_blocks(torch.from_numpy(vals[None, :]))
    assert int(sc[0, 0]) == 127
    dec = formats.dequant_fp4_blocks(packed.numpy(), sc.numpy())[0, :8]
    assert dec.tolist() == [4.0, 0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
