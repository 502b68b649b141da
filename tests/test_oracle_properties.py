"""Property tests of the oracle over small random shapes (hypothesis): the
top-k against a brute-force sort under ties, softmax weights with the sink
summing to one, and top-k >= eligible entries reducing CSA to dense attention
over entries + window."""
import numpy as np
import torch
import torch.nn.functional as F
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import csa

SETTINGS = settings(max_examples=40, deadline=None)


@SETTINGS
@given(n=st.integers(1, 40), k=st.integers(1, 48), levels=st.integers(1, 6), seed=st.integers(0, 2**31 - 1))
def test_topk_matches_sorted_with_lowest_index_ties(n, k, levels, seed):
    rng = np.random.default_rng(seed)
    scores = rng.integers(0, levels, size=n + 5).astype(np.float64)   # many ties
    got = csa.topk(scores, n, k)
    order = sorted(range(n), key=lambda j: (-scores[j], j))[:min(k, n)]
    want = np.array(sorted(order) + [-1] * (k - min(k, n)))
    assert np.array_equal(got, want)


@SETTINGS
@given(nkeys=st.integers(0, 12), d=st.sampled_from([2, 4, 8]), H=st.integers(1, 4),
       sink=st.floats(-4, 4), seed=st.integers(0, 2**31 - 1))
def test_weights_with_sink_sum_to_one(nkeys, d, H, sink, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, d))
    keys, vals = rng.standard_normal((nkeys, d)), rng.standard_normal((nkeys, d))
    out, lse, w, w_sink = csa.attend_keyset(q, keys, vals, np.full(H, sink), 0.7, return_weights=True)
    np.testing.assert_allclose(w.sum(axis=-1) + w_sink, 1.0, rtol=1e-12)
    np.testing.assert_allclose(w_sink, np.exp(sink - lse), rtol=1e-12)
    np.testing.assert_allclose(out, w @ vals, rtol=1e-12, atol=1e-14)


@SETTINGS
@given(T=st.integers(8, 40), m=st.integers(1, 4), window=st.integers(1, 6),
       seed=st.integers(0, 2**31 - 1))
def test_topk_covering_all_entries_is_dense_attention(T, m, window, seed):
    rng = np.random.default_rng(seed)
    d, H = 4, 2
    k, v = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    kc, vc, _ = csa.compress(k, v, None, rng.standard_normal(d), m)
    t = T - 1
    ne = csa.n_eligible(t, m)
    q = rng.standard_normal((1, H, d))
    idx = np.arange(ne)[None, :] if ne > 0 else np.full((1, 1), -1)
    out, _ = csa.sparse_attend(q, kc, vc, idx, k, v, 0, [t], window, None, 0.5)
    lo = max(0, t - window + 1)
    keys = np.concatenate([kc[:ne], k[lo:t + 1]])
    vals = np.concatenate([vc[:ne], v[lo:t + 1]])
    ref = F.scaled_dot_product_attention(torch.from_numpy(q[0])[:, None, :],
                                         torch.from_numpy(keys)[None].expand(H, -1, -1),
                                         torch.from_numpy(vals)[None].expand(H, -1, -1), scale=0.5)
    np.testing.assert_allclose(out[0], ref[:, 0].numpy(), rtol=1e-10, atol=1e-12)
