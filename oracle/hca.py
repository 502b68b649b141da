"""HCA (Heavily Compressed Attention) oracle, fp64.

hyper.ai summary of DeepSeek-V4, "Method", HCA paragraph: every m' (>> m)
tokens are consolidated into one entry without overlap, and attention over
the compressed entries is dense (no selection).  The pooling is the same
softmax-gated form as CSA's (``oracle.csa.compress`` with its own gate g').
The pages give HCA a sliding-window branch too; it is an optional argument
here (window=0 leaves only the compressed entries and the sink).
"""
from __future__ import annotations

import numpy as np

from .csa import attend_keyset, window_rows


def hca_attend(q, kc, vc, m_hca, positions, sink, scale, kraw=None, vraw=None,
               raw_pos0=0, window=0, return_weights=False):
    """Dense attention of each query over the completed m'-blocks
    j < floor((t+1)/m') (plus an optional raw window) and the sink.

    q: [Tq, H, d] at absolute `positions`; kc, vc: [N', d].
    Returns out [Tq, H, d], lse [Tq, H].
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(kc, dtype=np.float64)
    vc = np.asarray(vc, dtype=np.float64)
    Tq, H, d = q.shape
    out = np.zeros((Tq, H, d))
    lse = np.zeros((Tq, H))
    wts = []
    R = 0 if kraw is None else kraw.shape[0]
    for i, t in enumerate(np.asarray(positions).tolist()):
        n = (t + 1) // m_hca
        if n > kc.shape[0]:
            raise ValueError("query sees more completed blocks than the cache holds")
        keys = [kc[:n]]
        vals = [vc[:n]]
        rows = window_rows(t, window, raw_pos0, R)
        if rows.size:
            keys.append(np.asarray(kraw, dtype=np.float64)[rows])
            vals.append(np.asarray(vraw, dtype=np.float64)[rows])
        res = attend_keyset(q[i], np.concatenate(keys), np.concatenate(vals), sink, scale,
                            return_weights)
        out[i], lse[i] = res[0], res[1]
        if return_weights:
            wts.append((res[2], res[3]))
    return (out, lse, wts) if return_weights else (out, lse)
