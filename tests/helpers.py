"""Shared test utilities: device handling, fp64 views, and the comparison
rules (tolerances and the top-k near-tie band)."""
from __future__ import annotations

import numpy as np
import torch

# Output tolerances: max-abs 1e-5 (fp32) / 2e-2 (bf16), plus a relative
# Frobenius bound and an lse bound that separate a right kernel from zeros.
TOL = {"f32": dict(abs=1e-5, rel=1e-6, lse=1e-5), "bf16": dict(abs=2e-2, rel=1e-2, lse=1e-3)}
BAND_REL = 1e-6     # near-tie band for index sets, relative to the row's max score


def dev():
    return torch.device("cuda:0")


def f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().double().cpu().numpy()


def to_dev(d: dict) -> dict:
    return {k: v.to(dev()) for k, v in d.items()}


def assert_close(got, ref, dtype: str, what: str = "", lse_got=None, lse_ref=None):
    got, ref = f64(got), np.asarray(ref, dtype=np.float64)
    t = TOL[dtype]
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else mx
    assert mx <= t["abs"], f"{what}: max abs err {mx:.3e} > {t['abs']}"
    assert rel <= t["rel"], f"{what}: rel Frobenius err {rel:.3e} > {t['rel']}"
    if lse_got is not None:
        lg, lr = f64(lse_got), np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lr)
        assert np.array_equal(np.isfinite(lg), fin), f"{what}: lse finiteness differs"
        le = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
        assert le <= t["lse"], f"{what}: lse max abs err {le:.3e} > {t['lse']}"
    return mx, rel


def bf16_ulp_ok(got, ref, ulps: float = 1.0, slack=0.0):
    """|got - ref| <= ulps * ulp_bf16(ref) + slack (ref in fp64, got a bf16
    value).  `slack` carries the fp32 accumulation bound of the producer."""
    got, ref = f64(got), np.asarray(ref, dtype=np.float64)
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    bad = np.abs(got - ref) > ulps * ulp + slack
    return int(bad.sum()), float((np.abs(got - ref) / ulp).max())


def pool_slack(x, m):
    """fp32 accumulation bound of a pooled block: m * 2^-24 * max|x| over the
    block's rows, per (block, column).  x: [T, d] fp64."""
    x = np.asarray(x, dtype=np.float64)
    nc = x.shape[0] // m
    return m * 2.0 ** -24 * np.abs(x[: nc * m].reshape(nc, m, -1)).max(axis=1)


def check_topk_row(got_row, scores, n_e: int, k: int, band_rel: float = BAND_REL):
    """The GPU index set G for one query against the oracle's fp64 scores:
    |G| = min(k, n_e), ascending, unique, eligible, -1 padded; every entry
    scoring above tau + band is in G and none scoring below tau - band is,
    where tau is the oracle's k-th largest score and band = band_rel * max.
    Returns True if G equals the oracle's exact set."""
    got_row = np.asarray(got_row)
    m = min(k, n_e)
    sel = got_row[:m]
    assert np.all(got_row[m:] == -1), "padding must be -1"
    assert np.all(sel >= 0) and (m == 0 or sel.max() < n_e), "index out of the eligible range"
    assert np.all(np.diff(sel) > 0), "indices must be strictly ascending"
    if n_e <= k:
        assert np.array_equal(sel, np.arange(n_e))
        return True
    s = np.asarray(scores, dtype=np.float64)[:n_e]
    tau = np.sort(s)[::-1][k - 1]
    band = band_rel * s.max()
    inside = np.zeros(n_e, dtype=bool)
    inside[sel] = True
    must = s > tau + band
    assert np.all(inside[must]), f"{int((must & ~inside).sum())} clear winners missing"
    assert not np.any(inside & (s < tau - band)), "a clear loser was selected"
    order = np.lexsort((np.arange(n_e), -s))
    return np.array_equal(np.sort(order[:k]), sel)
