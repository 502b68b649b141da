"""Encoders that turn drawn fp32 values into the FP8 / FP4 codes the indexer
consumes (input preparation, shared by both sides).

Formats (OCP 8-bit floating point spec; OCP Microscaling (MX) spec v1.0):
  * FP8 E4M3 "fn": 1 sign, 4 exponent (bias 7), 3 mantissa bits; max 448;
    S.1111.111 is NaN; no infinities.
  * FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
    {0, .5, 1, 1.5, 2, 3, 4, 6}.  Packed two per byte, the even element in the
    low nibble.
  * E8M0 block scale: an unsigned biased exponent, value 2^(E-127).

Scale choices (not fixed by the pages, which only say the indexer QK path is
FP4 and FP8 extends the dynamic range): FP8 per-row scale = amax/448;
FP4 per-32 block scale = 2^(floor(log2 amax) - 2), the MX convention.  Both
sides decode the same codes, so parity does not depend on these choices.
"""
from __future__ import annotations

import numpy as np
import torch

FP8_MAX = 448.0


def quant_fp8_rows(x: torch.Tensor):
    """x: float32 [..., n] -> (codes uint8 [..., n], scale float32 [...])."""
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax)).float()
    y = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _e2m1_codes(mag: np.ndarray) -> np.ndarray:
    # Round-to-nearest-even onto {0,.5,1,1.5,2,3,4,6} with saturation at 6.
    # A midpoint between codes c and c+1 goes to the even one of the two.
    c = np.zeros(mag.shape, dtype=np.uint8)
    for mid, odd_lower in ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
                           (2.5, False), (3.5, True), (5.0, False)):
        c += (mag >= mid) if odd_lower else (mag > mid)
    return c


def quant_fp4_blocks(x: torch.Tensor, block: int = 32):
    """x: float32 [..., n], n % 32 == 0 -> (packed uint8 [..., n/2],
    e8m0 uint8 [..., n/32])."""
    xn = x.float().numpy()
    shp = xn.shape
    n = shp[-1]
    assert n % block == 0 and n % 2 == 0
    out_codes = np.empty(shp[:-1] + (n // 2,), dtype=np.uint8)
    out_scale = np.empty(shp[:-1] + (n // block,), dtype=np.uint8)
    flat = xn.reshape(-1, n)
    oc = out_codes.reshape(-1, n // 2)
    osc = out_scale.reshape(-1, n // block)
    step = max(1, (1 << 22) // n)
    for r0 in range(0, flat.shape[0], step):
        xb = flat[r0:r0 + step].reshape(-1, n // block, block).astype(np.float32)
        amax = np.abs(xb).max(axis=-1)
        _, ex = np.frexp(amax)                     # amax = f * 2^ex, f in [0.5, 1)
        e = np.where(amax > 0, ex.astype(np.int32) - 1 - 2, -127)
        e = np.clip(e, -127, 127)
        osc[r0:r0 + step] = (e + 127).astype(np.uint8)
        y = xb / np.ldexp(np.float32(1.0), e)[..., None].astype(np.float32)
        mag = np.abs(y)
        code = _e2m1_codes(mag)
        code = code | np.where((y < 0) & (code > 0), np.uint8(8), np.uint8(0))
        code = code.reshape(-1, n)
        oc[r0:r0 + step] = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return torch.from_numpy(out_codes), torch.from_numpy(out_scale)


def quant_kv8(kc: torch.Tensor, vc: torch.Tensor):
    """Mixed-precision cache rows (BF16 RoPE dims, FP8 the rest).

    kc, vc: [..., d] values.  Key dims 0 .. d/2-1 become E4M3 codes with one
    power-of-two scale per row, dims d/2 .. d-1 stay bf16; value rows become
    E4M3 codes with one power-of-two scale per row.  Power-of-two scales
    (2^ceil(log2(amax/448))) make code * scale exactly representable in bf16.
    Returns (k8, krope, kscale, v8, vscale)."""
    def rows(x):
        x = x.float()
        amax = x.abs().amax(dim=-1)
        e = torch.ceil(torch.log2(torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))))
        scale = torch.exp2(e).float()
        y = (x / scale.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
        return y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), scale.contiguous()
    d = kc.shape[-1]
    k8, ks = rows(kc[..., : d // 2])
    v8, vs = rows(vc)
    krope = kc[..., d // 2:].to(torch.bfloat16).contiguous()
    return k8, krope, ks, v8, vs

