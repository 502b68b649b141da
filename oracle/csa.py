"""CSA (Compressed Sparse Attention) oracle, fp64.

Follows the hyper.ai summary of DeepSeek-V4 ("Method", CSA paragraph) and the
aiboss88 explainer ("Technical Principles", CSA bullet), with the concrete
readings stated per function.  All arrays are float64 numpy; one sequence at a
time unless a function says otherwise.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# Block compression (CSA: every m tokens -> one entry; HCA reuses it with m').
# --------------------------------------------------------------------------
def compress(x_k, x_v, x_ki, g, m, pos_bias=None):
    """Softmax-gated pooling of each complete m-token block.

    Reading: the pages say m tokens are compressed into one entry "using
    learnable compression weights and positional biases".  For block j with
    tokens i = jm .. jm+m-1:  a_i = k_i . g + b_(i-jm),  pi = softmax_i(a),
    Kc_j = sum_i pi_i k_i, Vc_j = sum_i pi_i v_i, KIc_j = sum_i pi_i kI_i.
    The gate reads the raw key row; one gate serves K, V and the indexer key.
    A trailing partial block is not emitted.

    x_k, x_v: [T, d]; x_ki: [T, dI] or None; g: [d]; pos_bias: [m] or None.
    Returns (Kc [T//m, d], Vc [T//m, d], KIc [T//m, dI] or None).
    """
    x_k = np.asarray(x_k, dtype=np.float64)
    x_v = np.asarray(x_v, dtype=np.float64)
    T, d = x_k.shape
    nc = T // m
    kb = x_k[: nc * m].reshape(nc, m, d)
    vb = x_v[: nc * m].reshape(nc, m, d)
    a = kb @ np.asarray(g, dtype=np.float64)                       # [nc, m]
    if pos_bias is not None:
        a = a + np.asarray(pos_bias, dtype=np.float64)[None, :]
    a = a - a.max(axis=1, keepdims=True)
    p = np.exp(a)
    p = p / p.sum(axis=1, keepdims=True)
    kc = np.einsum("jm,jmd->jd", p, kb)
    vc = np.einsum("jm,jmd->jd", p, vb)
    kic = None
    if x_ki is not None:
        x_ki = np.asarray(x_ki, dtype=np.float64)
        ib = x_ki[: nc * m].reshape(nc, m, x_ki.shape[1])
        kic = np.einsum("jm,jmd->jd", p, ib)
    return kc, vc, kic


def compress_window(x_k, x_v, x_ki, g, m, width, pos_bias=None):
    """Softmax-gated pooling over overlapping windows.

    Reading: the HCA paragraph of the hyper.ai summary singles HCA out as
    compressing without overlap, so CSA's windows may overlap; the page gives
    no width.  Entry j pools the `width` tokens that end where block j ends,
    t = (j+1)m - width + i for i = 0..width-1, skipping t < 0, with the gate
    a_i = k_t . g + b_i (b indexed by window position) and the same softmax
    pooling as `compress`.  width = m is `compress`; entry j still needs
    (j+1)m tokens.

    x_k, x_v: [T, d]; x_ki: [T, dI] or None; pos_bias: [width] or None.
    """
    x_k = np.asarray(x_k, dtype=np.float64)
    x_v = np.asarray(x_v, dtype=np.float64)
    gv = np.asarray(g, dtype=np.float64)
    T, d = x_k.shape
    nc = T // m
    bias = np.zeros(width) if pos_bias is None else np.asarray(pos_bias, dtype=np.float64)
    kc = np.zeros((nc, d))
    vc = np.zeros((nc, d))
    kic = None if x_ki is None else np.zeros((nc, np.asarray(x_ki).shape[1]))
    for j in range(nc):
        start = (j + 1) * m - width
        rows = [start + i for i in range(width) if start + i >= 0]
        a = np.array([x_k[t] @ gv + bias[t - start] for t in rows])
        p = np.exp(a - a.max())
        p /= p.sum()
        kc[j] = p @ x_k[rows]
        vc[j] = p @ x_v[rows]
        if kic is not None:
            kic[j] = p @ np.asarray(x_ki, dtype=np.float64)[rows]
    return kc, vc, kic


def n_eligible(t, m):
    """Entries visible to a query at absolute position t: completed blocks
    only, i.e. block j is visible once its last token jm+m-1 <= t."""
    return (np.asarray(t) + 1) // m


# --------------------------------------------------------------------------
# Lightning indexer + top-k.
# --------------------------------------------------------------------------
def indexer_scores(qi, w, kic):
    """Index score of every entry for every query.

    Reading (no formula on the pages): I[t, j] = sum_h w[t,h] * ReLU(qI[t,h] . KIc_j).
    qi: [Tq, HI, dI]; w: [Tq, HI]; kic: [N, dI]  ->  [Tq, N].
    Eligibility is applied by the caller (topk takes n_e).
    """
    qi = np.asarray(qi, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kic = np.asarray(kic, dtype=np.float64)
    dots = np.einsum("thc,nc->thn", qi, kic)
    return np.einsum("th,thn->tn", w, np.maximum(dots, 0.0))


def topk(scores_row, n_e, k):
    """The min(k, n_e) largest of scores_row[:n_e]; equal scores go to the
    lower index.  Returned ascending by index, padded with -1 to length k."""
    s = np.asarray(scores_row, dtype=np.float64)[:n_e]
    j = np.arange(n_e)
    order = np.lexsort((j, -s))           # primary: score descending; then index
    sel = np.sort(order[: min(k, n_e)])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.size] = sel
    return out


def kth_score(scores_row, n_e, k):
    """Score of the last selected entry (the k-th largest), or None if n_e == 0."""
    s = np.sort(np.asarray(scores_row, dtype=np.float64)[:n_e])[::-1]
    if s.size == 0:
        return None
    return s[min(k, s.size) - 1]


# --------------------------------------------------------------------------
# Attention over an explicit key set with a per-head sink logit.
# --------------------------------------------------------------------------
def attend_keyset(q_t, keys, vals, sink, scale, return_weights=False):
    """One query token, all heads, over one key set shared by the heads (MQA).

    Reading: one softmax over {selected entries} U {window tokens} U {sink};
    the sink is a per-head logit s_h with a zero value vector, so it only
    enlarges the denominator.  With l = scale * q.key:
        M = max(s_h, max l);  Z = exp(s_h - M) + sum exp(l - M)
        o = sum exp(l - M) v / Z;  lse = M + ln Z.
    An empty key set gives o = 0 and lse = s_h (or -inf without a sink).
    q_t: [H, d]; keys, vals: [n, d]; sink: [H] or None.
    """
    q_t = np.asarray(q_t, dtype=np.float64)
    H = q_t.shape[0]
    keys = np.asarray(keys, dtype=np.float64).reshape(-1, q_t.shape[1])
    vals = np.asarray(vals, dtype=np.float64).reshape(-1, keys.shape[1] if keys.size else q_t.shape[1])
    logits = scale * (q_t @ keys.T)                                  # [H, n]
    if sink is None:
        s = np.full(H, -np.inf)
    else:
        s = np.asarray(sink, dtype=np.float64)
    lmax = logits.max(axis=1) if logits.shape[1] else np.full(H, -np.inf)
    M = np.maximum(s, lmax)
    if np.all(np.isneginf(M)):
        out = np.zeros((H, vals.shape[1]))
        lse = np.full(H, -np.inf)
        w = np.zeros((H, logits.shape[1]))
        return (out, lse, w, np.zeros(H)) if return_weights else (out, lse)
    Ms = np.where(np.isneginf(M), 0.0, M)
    e = np.exp(logits - Ms[:, None])
    es = np.exp(s - Ms)
    Z = e.sum(axis=1) + es
    out = (e @ vals) / np.where(Z > 0, Z, 1.0)[:, None]
    with np.errstate(divide="ignore"):
        lse = Ms + np.log(Z)
    if return_weights:
        return out, lse, e / Z[:, None], es / Z
    return out, lse


def window_rows(t, window, raw_pos0, R):
    """Row numbers (into a raw K/V buffer whose row r is absolute position
    raw_pos0 + r) of the sliding window of the query at position t:
    positions max(0, t-window+1) .. t, the query's own token included."""
    if window <= 0:
        return np.zeros(0, dtype=np.int64)
    lo = max(0, t - window + 1)
    rows = np.arange(lo, t + 1) - raw_pos0
    if rows.size and (rows[0] < 0 or rows[-1] >= R):
        raise ValueError("window reaches outside the raw K/V buffer")
    return rows


def sparse_attend(q, kc, vc, idx, kraw, vraw, raw_pos0, positions, window, sink, scale,
                  return_weights=False):
    """CSA core attention for one sequence.

    q: [Tq, H, d] queries at absolute positions `positions` [Tq];
    kc, vc: [N, d] compressed entries; idx: [Tq, k] selected entries (-1 = none);
    kraw, vraw: [R, d] raw tokens, row r at position raw_pos0 + r.
    The window is not de-duplicated against entries covering the same tokens.
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
        sel = np.asarray(idx[i])
        sel = sel[sel >= 0]
        rows = window_rows(t, window, raw_pos0, R)
        keys = [kc[sel]]
        vals = [vc[sel]]
        if rows.size:
            keys.append(np.asarray(kraw, dtype=np.float64)[rows])
            vals.append(np.asarray(vraw, dtype=np.float64)[rows])
        res = attend_keyset(q[i], np.concatenate(keys), np.concatenate(vals), sink, scale,
                            return_weights)
        out[i], lse[i] = res[0], res[1]
        if return_weights:
            wts.append((res[2], res[3]))
    return (out, lse, wts) if return_weights else (out, lse)
