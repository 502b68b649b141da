"""GPU parity of csa_indexer_topk: index sets against the fp64 oracle's
scores under the near-tie band rule, for fp32/bf16 prefill (chained on the
GPU's own compressed keys) and bf16 / FP8 / FP4 decode."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, check_topk_row, dev, f64
from oracle import formats
from sparse_attention_17_amd import ops
from synth import configs, inputs, quant

pytestmark = pytest.mark.gpu


def _dequant(x, name, qk):
    if qk == "fp8":
        return formats.dequant_fp8_rows(x[name].numpy(), x[name + "_scale"].numpy())
    if qk == "fp4":
        return formats.dequant_fp4_blocks(x[name].numpy(), x[name + "_scale"].numpy())
    return f64(x[name])


def _check_rows(idx, qi64, w64, kic64, positions, m, k, sample=None):
    rows = range(len(positions)) if sample is None else sample
    exact = 0
    n = 0
    for t in rows:
        pos = int(positions[t])
        ne = min((pos + 1) // m, kic64.shape[0])
        sc = oracle.csa.indexer_scores(qi64[t:t + 1], w64[t:t + 1], kic64[:ne])[0]
        exact += check_topk_row(idx[t], sc, ne, k)
        n += 1
    return exact, n


def _prefill(w, return_scores=False):
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    _, _, kic = ops.compress(g["k"], g["v"], g["ki"], g["g"], w.m)
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=dev())
    res = ops.indexer_topk(g["qi"], g["w"], kic, pos0, w.m, w.topk, max_pos=w.ctx - 1,
                           return_scores=return_scores)
    torch.cuda.synchronize()
    return x, kic, res


def test_tiny_f32_prefill_all_rows():
    w = configs.TINY
    x, kic, (idx, sc) = _prefill(w, return_scores=True)
    idx = idx.cpu().numpy()
    exact, n = _check_rows(idx[0], f64(x["qi"][0]), f64(x["w"][0]), f64(kic[0]),
                           np.arange(w.ctx), w.m, w.topk)
    assert exact == n          # fp32 ties this far apart: the sets must match exactly
    # returned scores line up with the returned indices
    s = sc.cpu().numpy()[0]
    ref = oracle.csa.indexer_scores(f64(x["qi"][0]), f64(x["w"][0]), f64(kic[0]))
    for t in (200, 700, 1023):
        ne = (t + 1) // w.m
        sel = idx[0, t][idx[0, t] >= 0]
        np.testing.assert_allclose(s[t, :sel.size], ref[t, sel], rtol=1e-5, atol=1e-7)
        assert np.all(np.isneginf(s[t, sel.size:]))
        assert ne >= sel.size


@pytest.mark.parametrize("HI,dI,k", [(4, 64, 512), (2, 32, 100), (1, 64, 64)])
def test_bf16_prefill_slice(HI, dI, k):
    w = configs.CSA_PREFILL_32K.with_(ctx=4096, Tq=4096, HI=HI, dI=dI, topk=k)
    x, kic, idx = _prefill(w)
    idx = idx.cpu().numpy()
    sample = list(range(0, 16)) + list(range(2040, 2056)) + list(range(4080, 4096)) + \
        list(np.random.default_rng(0).integers(0, 4096, 64))
    exact, n = _check_rows(idx[0], f64(x["qi"][0]), f64(x["w"][0]), f64(kic[0]),
                           np.arange(w.ctx), w.m, w.topk, sample)
    assert exact >= n - 2


def _decode(w):
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1,
                           qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                           qk_dtype=w.qk_dtype)
    torch.cuda.synchronize()
    return x, idx.cpu().numpy()


def _check_decode(w, x, idx):
    qi = _dequant(x, "qi", w.qk_dtype)
    kic = _dequant(x, "kic", w.qk_dtype)
    exact = 0
    for b in range(w.B):
        exact += _check_rows(idx[b], qi[b], f64(x["w"][b]), kic[b], [w.ctx - 1], w.m, w.topk)[0]
    return exact


@pytest.mark.parametrize("qk", ["bf16", "fp8", "fp4"])
def test_decode_small(qk):
    w = configs.HYBRID_1M_FP8.with_(ctx=65536 * 4, B=2, qk_dtype=qk, topk=2048)
    x, idx = _decode(w)
    assert _check_decode(w, x, idx) >= w.B - 1


def test_decode_csa_128k_full():
    w = configs.CSA_DECODE_128K
    x, idx = _decode(w)
    assert _check_decode(w, x, idx) >= w.B - 2


@pytest.mark.parametrize("qk", ["fp8", "fp4"])
def test_decode_hybrid_1m_full(qk):
    w = configs.HYBRID_1M_FP8.with_(qk_dtype=qk)
    x, idx = _decode(w)
    assert _check_decode(w, x, idx) >= w.B - 1


def test_padding_when_fewer_eligible_than_k():
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 1000, B=3, topk=4096)
    x, idx = _decode(w)
    assert np.all(idx[:, 0, :1000] == np.arange(1000)) and np.all(idx[:, 0, 1000:] == -1)


def test_ragged_positions_per_sequence():
    # sequences at different positions: each row sees its own eligible prefix
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 3000, B=3, topk=256)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos = [4 * 3000 - 1, 4 * 700 + 2, 5]
    pos0 = torch.tensor(pos, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, 4, 256, max_pos=max(pos))
    idx = idx.cpu().numpy()
    for b in range(3):
        _check_rows(idx[b], f64(x["qi"][b]), f64(x["w"][b]), f64(x["kic"][b]), [pos[b]], 4, 256)


@pytest.mark.parametrize("qk", ["bf16", "fp8"])
def test_long_rows_ragged_positions(qk):
    # long rows at different positions: rows whose chunk count and per-chunk
    # slot capacity differ from those of the last allowed position, and a row
    # with fewer eligible entries than k
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 40000, B=4, topk=1024, qk_dtype=qk)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos = [4 * 40000 - 1, 4 * 20000 + 1, 4 * 13000, 4 * 900 + 3]
    pos0 = torch.tensor(pos, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=max(pos),
                           qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                           qk_dtype=qk).cpu().numpy()
    qi = _dequant(x, "qi", qk)
    kic = _dequant(x, "kic", qk)
    exact = 0
    for b in range(w.B):
        exact += _check_rows(idx[b], qi[b], f64(x["w"][b]), kic[b], [pos[b]], w.m, w.topk)[0]
    assert exact >= w.B - 1
    assert np.all(idx[3, 0, :901] == np.arange(901)) and np.all(idx[3, 0, 901:] == -1)


def test_long_rows_all_tied_fall_back_exactly():
    # every score is 0: the boundary bin holds the whole row, which overflows the
    # candidate buffer; the exact fallback must return the lowest indices
    w = configs.CSA_DECODE_128K.with_(B=2)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    idx, sc = ops.indexer_topk(g["qi"], g["w"], torch.zeros_like(g["kic"]), pos0, w.m, w.topk,
                               max_pos=w.ctx - 1, return_scores=True)
    assert torch.equal(idx.cpu(), torch.arange(w.topk, dtype=torch.int32).expand(w.B, 1, -1))
    assert torch.all(sc == 0)


def test_long_rows_boundary_ties_take_lowest_indices():
    # 100 distinct key rows repeated over 32768 entries: every score value has
    # ~330 copies, so the k-th value is tied and the lowest indices must win
    w = configs.CSA_DECODE_128K.with_(B=2, topk=1000)
    x = inputs.make_inputs(w)
    base = x["kic"][:, :100]
    kic = base.repeat(1, w.Nc // 100 + 1, 1)[:, :w.Nc].contiguous()
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], kic.to(dev()), pos0, w.m, w.topk, max_pos=w.ctx - 1)
    idx = idx.cpu().numpy()
    for b in range(w.B):
        sc = oracle.csa.indexer_scores(f64(x["qi"][b]), f64(x["w"][b]), f64(kic[b]))[0]
        assert check_topk_row(idx[b, 0], sc, w.Nc, w.topk, band_rel=0.0)


def test_fp32_and_bf16_long_rows():
    for qk in ("f32", "bf16"):
        w = configs.CSA_DECODE_128K.with_(B=3, ctx=4 * 20000, qk_dtype=qk, topk=777)
        x, idx = _decode(w)
        assert _check_decode(w, x, idx) >= w.B - 1


# ---- prefill rows through the fused score+select kernel (no scores returned) ----

def _prefill_raw(B, Tq, HI, dI, Nc_cap, qk, wid):
    """Seeded qI / w / KIc for prefill rows that start at arbitrary positions."""
    qi = inputs.normal(wid, "qi", (B, Tq, HI, dI))
    kic = inputs.normal(wid, "kic", (B, Nc_cap, dI))
    wl = inputs.normal(wid, "wlog", (B, Tq, HI), scaled_by_last=False)
    x = {"w": torch.softmax(wl, dim=-1)}
    for name, v in (("qi", qi), ("kic", kic)):
        if qk == "fp8":
            x[name], x[name + "_scale"] = quant.quant_fp8_rows(v)
        elif qk == "fp4":
            x[name], x[name + "_scale"] = quant.quant_fp4_blocks(v)
        else:
            x[name] = inputs.to_dtype(v, qk)
    return x


def _check_all_prefill(x, idx, pos0, m, k, qk, band_rel=None):
    qi = _dequant(x, "qi", qk)
    kic = _dequant(x, "kic", qk)
    w64 = f64(x["w"])
    for b in range(idx.shape[0]):
        for t in range(idx.shape[1]):
            ne = min((pos0[b] + t + 1) // m, kic.shape[1])
            sc = oracle.csa.indexer_scores(qi[b, t:t + 1], w64[b, t:t + 1], kic[b, :ne])[0]
            kw = {} if band_rel is None else {"band_rel": band_rel}
            check_topk_row(idx[b, t], sc, ne, k, **kw)


def test_tiny_f32_fused_equals_score_then_select():
    # the same rows through both prefill paths: fp32 sets must be identical
    w = configs.TINY
    x, kic, (idx_a, _) = _prefill(w, return_scores=True)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=dev())
    idx_b = ops.indexer_topk(g["qi"], g["w"], kic, pos0, w.m, w.topk, max_pos=w.ctx - 1)
    assert torch.equal(idx_a, idx_b)


@pytest.mark.parametrize("qk,HI,dI,k", [("bf16", 2, 64, 128), ("fp8", 4, 64, 300),
                                        ("fp4", 1, 64, 64), ("f32", 4, 32, 512)])
def test_prefill_ragged_positions_and_tail(qk, HI, dI, k):
    # Tq not a multiple of the 16-token tile, sequences at different offsets
    B, Tq, Nc_cap, m = 2, 1000, 1024, 4
    pos = [3000, 17]
    x = _prefill_raw(B, Tq, HI, dI, Nc_cap, qk, 90 + HI)
    g = {n: v.to(dev()) for n, v in x.items()}
    pos0 = torch.tensor(pos, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, m, k, max_pos=pos[0] + Tq - 1,
                           qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                           qk_dtype=qk)
    _check_all_prefill(x, idx.cpu().numpy(), pos, m, k, qk)


def test_prefill_all_tied_rows():
    # every score is 0: rows with up to 512 eligible entries resolve the tied
    # boundary bin in LDS, longer rows overflow it and take the exact fallback;
    # both must return the lowest indices
    w = configs.CSA_PREFILL_32K.with_(ctx=4096, Tq=4096, topk=100)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    kic = torch.zeros(w.B, w.Nc, w.dI, dtype=torch.bfloat16, device=dev())
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], kic, pos0, w.m, w.topk, max_pos=w.ctx - 1).cpu()
    for t in range(w.Tq):
        ne = (t + 1) // w.m
        n = min(ne, w.topk)
        assert torch.equal(idx[0, t, :n], torch.arange(n, dtype=torch.int32)), t
        assert torch.all(idx[0, t, n:] == -1), t


def test_prefill_boundary_ties_take_lowest_indices():
    # 7 distinct key rows repeated: every score value has ~ne/7 copies, so the
    # k-th value is tied in every row; the lowest tied indices must win
    w = configs.CSA_PREFILL_32K.with_(ctx=4096, Tq=4096, topk=200, HI=2)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    base = inputs.normal(95, "kic", (w.B, 7, w.dI)).to(torch.bfloat16)
    kic = base.repeat(1, w.Nc // 7 + 1, 1)[:, :w.Nc].contiguous()
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], kic.to(dev()), pos0, w.m, w.topk,
                           max_pos=w.ctx - 1).cpu().numpy()
    qi, w64, k64 = f64(x["qi"][0]), f64(x["w"][0]), f64(kic[0])
    for t in list(range(790, 830)) + list(range(2040, 2060)) + list(range(4060, 4096)):
        ne = (t + 1) // w.m
        sc = oracle.csa.indexer_scores(qi[t:t + 1], w64[t:t + 1], k64[:ne])[0]
        assert check_topk_row(idx[0, t], sc, ne, w.topk, band_rel=0.0), t


@pytest.mark.parametrize("qk", ["bf16", "fp8", "fp4"])
def test_multi_token_decode_long_rows(qk):
    # three query tokens per sequence (the last three positions), long rows:
    # each token sees its own eligible prefix; then the sparse attention
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 40000 + 2, B=2, Tq=3, topk=1024, qk_dtype=qk)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 3, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1,
                           qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"), qk_dtype=qk)
    # the raw buffer holds the last `window` tokens: a window two shorter fits
    # every one of the three queries
    win = w.window - 2
    rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev())
    out, lse = ops.sparse_attend(g["q"], g["kc"], g["vc"], idx, pos0, w.ctx - 1, win,
                                 kw=g["kw"], vw=g["vw"], raw_pos0=rp0, sink=g["sink"],
                                 return_lse=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    qi, kic = _dequant(x, "qi", qk), _dequant(x, "kic", qk)
    positions = list(range(w.ctx - 3, w.ctx))
    exact = 0
    for b in range(w.B):
        exact += _check_rows(idx[b], qi[b], f64(x["w"][b]), kic[b], positions, w.m, w.topk)[0]
        ro, rl = oracle.csa.sparse_attend(f64(x["q"][b]), f64(x["kc"][b]), f64(x["vc"][b]), idx[b],
                                          f64(x["kw"][b]), f64(x["vw"][b]), w.ctx - w.window,
                                          positions, win, f64(x["sink"]), w.scale)
        assert_close(out[b], ro, "bf16", f"attend[{b}]", lse[b], rl)
    assert exact >= 3 * w.B - 1


@pytest.mark.parametrize("qk", ["fp8", "fp4", "bf16"])
def test_decode_score_accuracy(qk):
    # the decode score kernels' fp32 scores of the selected entries against the
    # oracle's fp64 scores of the same decoded values: the error must stay far
    # inside the 1e-6 near-tie band (relative to the row maximum), so that the
    # index sets are exact outside it
    w = configs.HYBRID_1M_FP8.with_(ctx=65536 * 4, B=2, qk_dtype=qk, topk=2048)
    x = inputs.make_inputs(w, peaky=True)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    idx, sc = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1,
                               qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                               qk_dtype=qk, return_scores=True)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    qi = _dequant(x, "qi", qk)
    kic = _dequant(x, "kic", qk)
    worst = 0.0
    for b in range(w.B):
        ref = oracle.csa.indexer_scores(qi[b], f64(x["w"][b]), kic[b])[0]
        sel = idx[b, 0]
        rel = np.abs(sc[b, 0] - ref[sel]).max() / ref.max()
        worst = max(worst, rel)
    print(f"decode {qk} score error: {worst:.2e} of the row maximum")
    assert worst < 3e-7                     # the band is 1e-6; native FP8 MFMA sums measured ~1e-5
