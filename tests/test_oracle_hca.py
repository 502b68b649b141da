"""Pins for the oracle's HCA attention: m'=1 with no window and no sink is
textbook causal attention (PyTorch SDPA, float64); completed-block
eligibility at m'>1 maps onto causal attention over the compressed sequence;
the empty key set leaves only the sink."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import csa, hca


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, **kw):
    H = q.shape[1]
    out = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).expand(H, -1, -1),
        torch.from_numpy(v).expand(H, -1, -1), scale=scale, **kw)
    return out.permute(1, 0, 2).numpy()


def test_m1_no_sink_is_causal_sdpa():
    T, H, d = 40, 4, 8
    k, v, q = _rand((T, d), 0), _rand((T, d), 1), _rand((T, H, d), 2)
    kc, vc, _ = csa.compress(k, v, None, _rand(d, 3), 1)
    out, _ = hca.hca_attend(q, kc, vc, 1, np.arange(T), None, 0.35)
    np.testing.assert_allclose(out, _sdpa(q, k, v, 0.35, is_causal=True), rtol=1e-12, atol=1e-14)


def test_m1_with_sink_is_sdpa_with_sink_column():
    T, H, d = 24, 3, 8
    k, v, q = _rand((T, d), 4), _rand((T, d), 5), _rand((T, H, d), 6)
    sink = _rand(H, 7)
    out, lse = hca.hca_attend(q, k, v, 1, np.arange(T), sink, 0.5)
    K = np.concatenate([np.zeros((1, d)), k])
    V = np.concatenate([np.zeros((1, d)), v])
    mask = np.full((H, T, T + 1), -np.inf)
    for t in range(T):
        mask[:, t, 0] = sink
        mask[:, t, 1:t + 2] = 0.0
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(K).expand(H, -1, -1),
        torch.from_numpy(V).expand(H, -1, -1), attn_mask=torch.from_numpy(mask), scale=0.5)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-14)
    # lse against a direct log-sum-exp of the same logits
    lg = 0.5 * np.einsum("thd,jd->thj", q, k)
    for t in range(T):
        z = np.exp(sink) + np.exp(lg[t, :, : t + 1]).sum(axis=1)
        np.testing.assert_allclose(lse[t], np.log(z), rtol=1e-13)


@pytest.mark.parametrize("mp", [4, 32])
def test_completed_block_eligibility(mp):
    nb, H, d = 12, 2, 8
    T = nb * mp
    kc, vc = _rand((nb, d), 8), _rand((nb, d), 9)
    qc = _rand((nb, H, d), 10)
    ref = _sdpa(qc, kc, vc, 0.4, is_causal=True)       # query q sees entries 0..q
    # a query at t = mp*q + mp - 1 has just completed block q
    out, _ = hca.hca_attend(qc, kc, vc, mp, mp * np.arange(nb) + mp - 1, None, 0.4)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # one token earlier, block q is still open: entries 0..q-1
    out2, _ = hca.hca_attend(qc[1:], kc, vc, mp, mp * np.arange(1, nb) + mp - 2, None, 0.4)
    ref2 = _sdpa(qc[1:], kc[:-1], vc[:-1], 0.4, is_causal=True)
    np.testing.assert_allclose(out2, ref2, rtol=1e-12, atol=1e-14)
    assert T == nb * mp


def test_empty_key_set_leaves_the_sink():
    H, d = 3, 8
    kc, vc, q = _rand((4, d), 11), _rand((4, d), 12), _rand((5, H, d), 13)
    sink = _rand(H, 14)
    out, lse = hca.hca_attend(q, kc, vc, 32, np.arange(5), sink, 0.3)
    assert np.all(out == 0)
    np.testing.assert_array_equal(lse, np.broadcast_to(sink, lse.shape))
    out, lse = hca.hca_attend(q, kc, vc, 32, np.arange(5), None, 0.3)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_cache_too_small_is_an_error():
    with pytest.raises(ValueError):
        hca.hca_attend(_rand((1, 2, 8), 0), _rand((3, 8), 1), _rand((3, 8), 2), 4, [15], None, 1.0)
