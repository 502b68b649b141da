"""Exact decoders for the indexer's low-precision formats (fp64 results).

Definitions (not from the DeepSeek-V4 pages, which only state that the
indexer QK path is FP4 and that FP8 extends its dynamic range — aiboss88
"Technical Principles", FP4 bullet; hyper.ai "Method", efficiency paragraph):
  * OCP 8-bit floating point spec, E4M3 ("fn" variant): exponent bias 7,
    normal = (-1)^s 2^(e-7) (1 + f/8), subnormal (e=0) = (-1)^s 2^-6 f/8,
    S.1111.111 = NaN, no infinities.
  * OCP MX spec v1.0, E2M1: exponent bias 1, normal = (-1)^s 2^(e-1) (1 + f/2),
    subnormal (e=0) = (-1)^s f/2.  E8M0 scale: 2^(E-127), E=255 is NaN.
FP4 data is packed two per byte with the even-indexed element in the low
nibble.
"""
from __future__ import annotations

import numpy as np


def e4m3_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    f = (c & 7).astype(np.float64)
    normal = (1.0 + f / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (f / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (c & 7 == 7), np.nan, val)
    return np.where(s == 1, -val, val)


def e2m1_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    f = (c & 1).astype(np.float64)
    normal = (1.0 + f / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    sub = f / 2.0
    val = np.where(e == 0, sub, normal)
    return np.where(s == 1, -val, val)


def e8m0_to_f64(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def unpack_fp4(packed) -> np.ndarray:
    """uint8 [..., n/2] -> nibble codes [..., n]; element 2i is the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def dequant_fp8_rows(codes, scale) -> np.ndarray:
    """codes uint8 [..., n] with one fp32 scale per row [...] -> fp64 [..., n]."""
    return e4m3_to_f64(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def dequant_fp4_blocks(packed, scales, block: int = 32) -> np.ndarray:
    """packed uint8 [..., n/2], E8M0 scales uint8 [..., n/block] -> fp64 [..., n]."""
    vals = e2m1_to_f64(unpack_fp4(packed))
    n = vals.shape[-1]
    vb = vals.reshape(vals.shape[:-1] + (n // block, block))
    vb = vb * e8m0_to_f64(scales)[..., None]
    return vb.reshape(vals.shape)
