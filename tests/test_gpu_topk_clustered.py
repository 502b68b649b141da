"""Long decode rows whose top-k entries cluster at the end of the row (the most
recent 5 % of the compressed entries score higher), the case where the
per-chunk candidate cut cannot hold a chunk's share of the top-k.  The index
sets must still match the fp64 oracle under the near-tie band (aiboss88
"Technical Principles", CSA bullet: top-k sparse selection by index score);
the selection takes the second round over the unsafe chunks' stored scores
instead of the single-workgroup exact select."""
import numpy as np
import pytest
import torch

import oracle
from helpers import check_topk_row, dev, f64
from oracle import formats
from sparse_attention_17_amd import ops
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def _clustered(qk, B):
    w = configs.HYBRID_1M_FP8.with_(B=B, qk_dtype=qk)          # 262,144 entries, top-2048
    x = inputs.make_inputs(w)
    hot = w.Nc - w.Nc // 20
    if qk == "fp8":
        x["kic_scale"][:, hot:] *= 3.0                          # the last 5 % of keys three times larger
        kic64 = formats.dequant_fp8_rows(x["kic"].numpy(), x["kic_scale"].numpy())
        qi64 = formats.dequant_fp8_rows(x["qi"].numpy(), x["qi_scale"].numpy())
    else:
        x["kic"][:, hot:] = (x["kic"][:, hot:].float() * 3.0).to(x["kic"].dtype)
        kic64, qi64 = f64(x["kic"]), f64(x["qi"])
    return w, x, qi64, kic64


@pytest.mark.parametrize("qk", ["bf16", "fp8"])
def test_clustered_topk_second_round(qk):
    w, x, qi64, kic64 = _clustered(qk, 2)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    ops.profile_counter("indexer_decode_second_round", reset=True)
    ops.profile_counter("indexer_decode_fallback", reset=True)
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1,
                           qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"), qk_dtype=qk)
    idx = idx.cpu().numpy()
    rounds = ops.profile_counter("indexer_decode_second_round", reset=True)
    fallback = ops.profile_counter("indexer_decode_fallback", reset=True)
    hot = w.Nc - w.Nc // 20
    for b in range(w.B):
        sc = oracle.csa.indexer_scores(qi64[b], f64(x["w"][b]), kic64[b])[0]
        check_topk_row(idx[b, 0], sc, w.Nc, w.topk)
        assert np.mean(idx[b, 0] >= hot) > 0.5                  # the selection is indeed clustered
    print(f"clustered {qk}: second rounds {rounds}, exact fallbacks {fallback} of {w.B} rows")
    assert rounds == w.B and fallback == 0


def test_clustered_topk_in_the_fused_step():
    # the same rows through the decode step, with and without the fused tail
    w, x, qi64, kic64 = _clustered("fp8", 8)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev())
    idx = dict(qi=g["qi"], w=g["w"], kic=g["kic"], m=w.m, topk=w.topk, qi_scale=g["qi_scale"],
               kic_scale=g["kic_scale"], qk_dtype="fp8")
    csa = dict(q=g["q"], kc=g["kc"], vc=g["vc"], window=w.window, kw=g["kw"], vw=g["vw"],
               raw_pos0=rp0, sink=g["sink"])
    hca = dict(q=g["q_hca"], kc=g["kc_hca"], vc=g["vc_hca"], m_prime=w.m_hca, sink=g["sink_hca"])
    ops.profile_counter("step_timeout", reset=True)
    fused = ops.DecodeStep(idx, csa, hca, pos0, w.ctx - 1, fused_tail=True).run()
    sep = ops.DecodeStep(idx, csa, hca, pos0, w.ctx - 1).run()
    torch.cuda.synchronize()
    assert torch.equal(fused.idx, sep.idx)
    assert torch.equal(fused.out.view(torch.int16), sep.out.view(torch.int16))
    assert ops.profile_counter("step_timeout", reset=True) == 0
    got = fused.idx.cpu().numpy()
    for b in (0, w.B - 1):
        sc = oracle.csa.indexer_scores(qi64[b], f64(x["w"][b]), kic64[b])[0]
        check_topk_row(got[b, 0], sc, w.Nc, w.topk)
