"""Pins for the oracle's CSA attention: when top-k keeps every eligible entry
it must equal dense attention (PyTorch SDPA in float64) over entries + window
+ a sink column; weights sum to one with the sink; limits of the sink; the
window alone reduces to causal attention over raw tokens."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import csa


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_with_sink(q_t, keys, vals, sink, scale):
    """Dense reference: a zero key/value column whose logit is the sink."""
    H, d = q_t.shape
    K = torch.from_numpy(np.concatenate([np.zeros((1, d)), keys]))
    V = torch.from_numpy(np.concatenate([np.zeros((1, d)), vals]))
    mask = torch.zeros(H, 1, K.shape[0], dtype=torch.float64)
    mask[:, 0, 0] = torch.from_numpy(np.asarray(sink, dtype=np.float64))
    q = torch.from_numpy(q_t).reshape(H, 1, d)
    out = F.scaled_dot_product_attention(q, K.expand(H, -1, -1), V.expand(H, -1, -1),
                                         attn_mask=mask, scale=scale)
    return out.reshape(H, d).numpy()


def _setup(seed, T=48, d=16, H=3, m=4, W=6):
    k, v = _rand((T, d), seed) / 4, _rand((T, d), seed + 1) / 4
    kc, vc, _ = csa.compress(k, v, None, _rand(d, seed + 2), m)
    q = _rand((T, H, d), seed + 3)
    sink = _rand(H, seed + 4)
    return k, v, kc, vc, q, sink


@pytest.mark.parametrize("W", [0, 1, 6, 48])
def test_full_topk_equals_dense_attention_with_sink(W):
    k, v, kc, vc, q, sink = _setup(0, W=W)
    T, H, d = q.shape
    m, scale = 4, 0.3
    pos = np.arange(T)
    idx = np.full((T, kc.shape[0]), -1, dtype=np.int32)
    for t in range(T):
        idx[t, : csa.n_eligible(t, m)] = np.arange(csa.n_eligible(t, m))
    out, lse = csa.sparse_attend(q, kc, vc, idx, k, v, 0, pos, W, sink, scale)
    for t in range(T):
        ne = csa.n_eligible(t, m)
        lo = max(0, t - W + 1)
        keys = np.concatenate([kc[:ne], k[lo:t + 1] if W else np.zeros((0, d))])
        vals = np.concatenate([vc[:ne], v[lo:t + 1] if W else np.zeros((0, d))])
        ref = sdpa_with_sink(q[t], keys, vals, sink, scale)
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-14)


def test_weights_sum_to_one_with_sink_and_lse():
    k, v, kc, vc, q, sink = _setup(10)
    T = q.shape[0]
    idx = np.stack([np.r_[np.arange(csa.n_eligible(t, 4)), -np.ones(12 - csa.n_eligible(t, 4))]
                    for t in range(T)]).astype(np.int32)
    out, lse, wts = csa.sparse_attend(q, kc, vc, idx, k, v, 0, np.arange(T), 6, sink, 0.25,
                                      return_weights=True)
    for t, (wk, ws) in enumerate(wts):
        np.testing.assert_allclose(wk.sum(axis=1) + ws, 1.0, rtol=0, atol=1e-14)
        # sink weight = exp(sink - lse)
        np.testing.assert_allclose(ws, np.exp(sink - lse[t]), rtol=1e-12)


def test_sink_limits():
    k, v, kc, vc, q, _ = _setup(20)
    T, H, d = q.shape
    idx = np.zeros((T, 1), dtype=np.int32) - 1
    pos = np.arange(T)
    no_sink, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, pos, 6, None, 0.3)
    very_neg, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, pos, 6, np.full(H, -800.0), 0.3)
    very_pos, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, pos, 6, np.full(H, 800.0), 0.3)
    np.testing.assert_allclose(very_neg, no_sink, rtol=1e-14, atol=0)
    assert np.abs(very_pos).max() < 1e-300


def test_window_only_is_causal_attention_over_raw_tokens():
    k, v, kc, vc, q, _ = _setup(30)
    T, H, d = q.shape
    idx = np.full((T, 4), -1, dtype=np.int32)
    out, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, np.arange(T), T, None, 0.3)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).expand(H, -1, -1),
        torch.from_numpy(v).expand(H, -1, -1), is_causal=True, scale=0.3)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)


def test_window_of_one_returns_own_value():
    k, v, kc, vc, q, _ = _setup(40)
    T = q.shape[0]
    idx = np.full((T, 2), -1, dtype=np.int32)
    out, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, np.arange(T), 1, None, 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, None, :], out.shape), rtol=1e-15)


def test_index_order_does_not_matter():
    k, v, kc, vc, q, sink = _setup(50)
    T = q.shape[0]
    rng = np.random.default_rng(0)
    idx = np.full((T, 8), -1, dtype=np.int32)
    for t in range(T):
        ne = csa.n_eligible(t, 4)
        sel = rng.permutation(ne)[:8]
        idx[t, : sel.size] = np.sort(sel)
    a, la = csa.sparse_attend(q, kc, vc, idx, k, v, 0, np.arange(T), 6, sink, 0.3)
    perm = idx[:, ::-1].copy()
    b, lb = csa.sparse_attend(q, kc, vc, perm, k, v, 0, np.arange(T), 6, sink, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-13)


def test_decode_window_offsets():
    # raw buffer holding only the last W tokens (row r at position raw_pos0 + r)
    k, v, kc, vc, q, sink = _setup(60)
    T, H, d = q.shape
    W = 6
    t = T - 1
    idx = np.arange(csa.n_eligible(t, 4), dtype=np.int32)[None, :]
    full, _ = csa.sparse_attend(q[t:], kc, vc, idx, k, v, 0, [t], W, sink, 0.3)
    tail, _ = csa.sparse_attend(q[t:], kc, vc, idx, k[T - W:], v[T - W:], T - W, [t], W, sink, 0.3)
    np.testing.assert_array_equal(full, tail)
    with pytest.raises(ValueError):
        csa.sparse_attend(q[t:], kc, vc, idx, k[T - W + 1:], v[T - W + 1:], T - W + 1, [t], W,
                          sink, 0.3)
