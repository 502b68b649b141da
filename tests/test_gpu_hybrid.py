"""csa_hybrid_attend: the CSA and HCA attention of one layer pair in one call.
Split decode runs as one fused launch, other shapes as the two calls in
sequence; either way outputs and lse are bitwise those of csa_sparse_attend +
hca_attend, match the fp64 oracle, repeat bitwise and do not depend on the
batch."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, dev, f64
from sparse_attention_17_amd import _lib as L
from sparse_attention_17_amd import ops
from synth import configs, inputs

pytestmark = pytest.mark.gpu

# 65536 CSA entries per sequence, 2048 HCA entries (m' = 128)
W = configs.HYBRID_1M_FP8.with_(ctx=4 * 65536, B=4)


def _setup(w, x, idx_np=None):
    g = {k: v.to(dev()) for k, v in x.items()}
    B = g["q"].shape[0]
    pos0 = torch.full((B,), w.ctx - 1, dtype=torch.int32, device=dev())
    rp0 = torch.full((B,), w.ctx - w.window, dtype=torch.int32, device=dev())
    if idx_np is None:
        idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1,
                               qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                               qk_dtype=w.qk_dtype)
    else:
        idx = torch.from_numpy(idx_np).to(dev())
    csa = dict(q=g["q"], kc=g["kc"], vc=g["vc"], idx=idx, pos0=pos0, max_pos=w.ctx - 1,
               window=w.window, kw=g["kw"], vw=g["vw"], raw_pos0=rp0, sink=g["sink"])
    hca = None
    if "q_hca" in g:
        hca = dict(q=g["q_hca"], kc=g["kc_hca"], vc=g["vc_hca"], m_prime=w.m_hca, pos0=pos0,
                   max_pos=w.ctx - 1, sink=g["sink_hca"])
    return csa, hca


def _separate(csa, hca):
    o1, l1 = ops.sparse_attend(**csa, return_lse=True)
    o2, l2 = ops.hca_attend(**hca, return_lse=True)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o1, l1, o2, l2)]


def _fused(csa, hca):
    res = ops.hybrid_attend(csa, hca, return_lse=True)
    torch.cuda.synchronize()
    return [t.cpu() for t in res]


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b):
    return all(torch.equal(_bits(u), _bits(v)) for u, v in zip(a, b))


def _pair_launches(fn):
    lib = L.load()
    lib.csa_profile_reset()
    lib.csa_profile_enable(1)
    fn()
    torch.cuda.synchronize()
    lib.csa_profile_enable(0)
    n, t = C.c_int(0), C.c_double(0)
    st = lib.csa_profile_query(b"attend_pair", C.byref(n), C.byref(t))
    lib.csa_profile_reset()
    return n.value if st == 0 else 0


def _check_oracle(x, w, got, idx, seqs, dtype):
    for b in seqs:
        ro, rl = oracle.csa.sparse_attend(f64(x["q"][b]), f64(x["kc"][b]), f64(x["vc"][b]),
                                          idx[b], f64(x["kw"][b]), f64(x["vw"][b]),
                                          w.ctx - w.window, [w.ctx - 1], w.window,
                                          f64(x["sink"]), w.scale)
        assert_close(got[0][b], ro, dtype, f"csa[{b}]", got[1][b], rl)


def _check_oracle_hca(x, w, got, seqs, dtype):
    for b in seqs:
        ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), f64(x["kc_hca"][b]),
                                       f64(x["vc_hca"][b]), w.m_hca, [w.ctx - 1],
                                       f64(x["sink_hca"]), w.scale)
        assert_close(got[2][b], ro, dtype, f"hca[{b}]", got[3][b], rl)


def test_decode_pair_is_one_launch_and_matches_oracle():
    x = inputs.make_inputs(W, peaky=True)
    csa, hca = _setup(W, x)
    got = []
    assert _pair_launches(lambda: got.extend(_fused(csa, hca))) == 1
    _check_oracle(x, W, got, csa["idx"].cpu().numpy(), range(W.B), W.dtype)
    _check_oracle_hca(x, W, got, range(W.B), W.dtype)
    assert _same(_separate(csa, hca), got)


def test_decode_pair_repeats_and_batch_invariance():
    x = inputs.make_inputs(W)
    csa, hca = _setup(W, x)
    full = _fused(csa, hca)
    assert _same(full, _fused(csa, hca))
    idx = csa["idx"].cpu()
    for b in (0, 3):
        xb = {k: (v[b:b + 1].contiguous() if v.dim() >= 2 and v.shape[0] == W.B else v)
              for k, v in x.items()}
        cb, hb = _setup(W.with_(B=1), xb, idx[b:b + 1].numpy())
        one = _fused(cb, hb)
        assert _same([t[b:b + 1] for t in full], one), f"sequence {b} differs at batch 1"


def test_decode_pair_with_different_batches_and_holes():
    # the CSA problem has 4 sequences with holes in its index lists, the HCA
    # problem 2 sequences at another position
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 6000, B=4, topk=1024)
    x = inputs.make_inputs(w, peaky=True)
    rng = np.random.default_rng(5)
    idx = np.stack([np.sort(rng.choice(6000, 1024, replace=False)) for _ in range(4)])
    idx = idx[:, None, :].astype(np.int32)
    idx[rng.random(idx.shape) < 0.2] = -1
    csa, _ = _setup(w, x, idx)
    wh = configs.HCA_1M_DECODE.with_(B=2, ctx=128 * 3000 + 77)
    xh = inputs.make_inputs(wh, peaky=True)
    gh = {k: v.to(dev()) for k, v in xh.items()}
    ph = torch.full((2,), wh.ctx - 1, dtype=torch.int32, device=dev())
    hca = dict(q=gh["q_hca"], kc=gh["kc_hca"], vc=gh["vc_hca"], m_prime=wh.m_hca, pos0=ph,
               max_pos=wh.ctx - 1, sink=gh["sink_hca"])
    got = []
    assert _pair_launches(lambda: got.extend(_fused(csa, hca))) == 1
    assert _same(_separate(csa, hca), got)
    _check_oracle(x, w, got, idx, range(4), w.dtype)
    _check_oracle_hca(xh, wh, got, range(2), wh.dtype)


def test_prefill_pair_runs_the_two_calls():
    # Tq > 1: no split, so the two problems run one after the other
    w = configs.TINY
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.zeros(1, dtype=torch.int32, device=dev())
    kc, vc, kic = ops.compress(g["k"], g["v"], g["ki"], g["g"], w.m)
    idx = ops.indexer_topk(g["qi"], g["w"], kic, pos0, w.m, w.topk, max_pos=w.ctx - 1)
    kh, vh, _ = ops.compress(g["k"], g["v"], None, g["g_hca"], w.m_hca)
    csa = dict(q=g["q"], kc=kc, vc=vc, idx=idx, pos0=pos0, max_pos=w.ctx - 1, window=w.window,
               kw=g["k"], vw=g["v"], raw_pos0=pos0, sink=g["sink"])
    hca = dict(q=g["q_hca"], kc=kh, vc=vh, m_prime=w.m_hca, pos0=pos0, max_pos=w.ctx - 1,
               sink=g["sink_hca"])
    ref = _separate(csa, hca)
    got = []
    assert _pair_launches(lambda: got.extend(_fused(csa, hca))) == 0
    assert _same(ref, got)


def test_f32_decode_pair():
    # fp32, 4 query heads: one decode token per sequence at the last position,
    # over caches compressed from the sequence; both problems split
    w = configs.TINY.with_(B=3, topk=256, m_hca=2)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    zero = torch.zeros(w.B, dtype=torch.int32, device=dev())
    kc, vc, kic = ops.compress(g["k"], g["v"], g["ki"], g["g"], w.m)
    kh, vh, _ = ops.compress(g["k"], g["v"], None, g["g_hca"], w.m_hca)
    q1 = g["q"][:, -1:].contiguous()
    qh = g["q_hca"][:, -1:].contiguous()
    idx = ops.indexer_topk(g["qi"][:, -1:].contiguous(), g["w"][:, -1:].contiguous(), kic, pos0,
                           w.m, w.topk, max_pos=w.ctx - 1)
    csa = dict(q=q1, kc=kc, vc=vc, idx=idx, pos0=pos0, max_pos=w.ctx - 1, window=w.window,
               kw=g["k"], vw=g["v"], raw_pos0=zero, sink=g["sink"])
    hca = dict(q=qh, kc=kh, vc=vh, m_prime=w.m_hca, pos0=pos0, max_pos=w.ctx - 1,
               sink=g["sink_hca"])
    got = []
    assert _pair_launches(lambda: got.extend(_fused(csa, hca))) == 1
    assert _same(_separate(csa, hca), got)
    kc64, vc64, kh64, vh64 = (f64(t.cpu()) for t in (kc, vc, kh, vh))
    idx64 = idx.cpu().numpy()
    for b in range(w.B):
        ro, rl = oracle.csa.sparse_attend(f64(x["q"][b, -1:]), kc64[b], vc64[b], idx64[b],
                                          f64(x["k"][b]), f64(x["v"][b]), 0, [w.ctx - 1],
                                          w.window, f64(x["sink"]), w.scale)
        assert_close(got[0][b], ro, "f32", f"csa[{b}]", got[1][b], rl)
        ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b, -1:]), kh64[b], vh64[b], w.m_hca,
                                       [w.ctx - 1], f64(x["sink_hca"]), w.scale)
        assert_close(got[2][b], ro, "f32", f"hca[{b}]", got[3][b], rl)


def test_decode_pair_hca_with_window():
    # the HCA problem with its own sliding window over raw rows
    w = configs.HYBRID_1M_FP8.with_(ctx=4 * 65536, B=2)
    x = inputs.make_inputs(w)
    csa, hca = _setup(w, x)
    hca.update(window=64, kw=csa["kw"], vw=csa["vw"], raw_pos0=csa["raw_pos0"])
    ref = _separate(csa, hca)
    got = []
    assert _pair_launches(lambda: got.extend(_fused(csa, hca))) == 1
    assert _same(ref, got)
    for b in range(w.B):
        ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), f64(x["kc_hca"][b]), f64(x["vc_hca"][b]),
                                       w.m_hca, [w.ctx - 1], f64(x["sink_hca"]), w.scale,
                                       kraw=f64(x["kw"][b]), vraw=f64(x["vw"][b]),
                                       raw_pos0=w.ctx - w.window, window=64)
        assert_close(got[2][b], ro, w.dtype, f"hca+window[{b}]", got[3][b], rl)

