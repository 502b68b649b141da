"""Grouped output projection oracle, fp64.

hyper.ai summary of DeepSeek-V4, "Method", CSA paragraph: the core attention
(MQA) is followed by a grouped output projection, there to keep the cost of
projecting many heads down.  The page names the operation only; the form
implemented (the plainest one it supports) splits the H heads into G
consecutive groups and gives each group its own projection matrix:

    y[t, j*dg:(j+1)*dg] = concat_{h in group j} o[t, h, :]  @  W_j^T

with W_j of shape [dg, (H/G)*d] (one row per output, as a linear layer's
weight is usually stored).  The groups are independent, so this is a plain
matrix product per group (numpy's matmul is the one library step).
"""
from __future__ import annotations

import numpy as np


def grouped_out_proj(o, w):
    """o: [T, H, d]; w: [G, dg, (H/G)*d]  ->  y: [T, G*dg] (fp64)."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, H, d = o.shape
    G, dg, K = w.shape
    assert H % G == 0 and K == (H // G) * d
    hg = H // G
    y = np.empty((T, G * dg))
    for j in range(G):
        heads = o[:, j * hg:(j + 1) * hg, :].reshape(T, K)    # the group's heads, concatenated
        y[:, j * dg:(j + 1) * dg] = heads @ w[j].T
    return y
