"""The decode step (indexer + top-k, then the paired CSA/HCA attention)
captured in a HIP graph: every replay, with eager work and synchronisations
between replays, reproduces the eager results bitwise.  The library records
no memset and allocates nothing, so its launches are capturable as they are."""
import pytest
import torch

from helpers import dev
from sparse_attention_17_amd import ops
from synth import configs, inputs

pytestmark = pytest.mark.gpu

W = configs.HYBRID_1M_FP8.with_(ctx=4 * 65536, B=4)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_captured_decode_step_replays_match_eager():
    x = inputs.make_inputs(W)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.full((W.B,), W.ctx - 1, dtype=torch.int32, device=dev())
    rp0 = torch.full((W.B,), W.ctx - W.window, dtype=torch.int32, device=dev())

    def step():
        idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, W.m, W.topk, max_pos=W.ctx - 1,
                               qi_scale=g.get("qi_scale"), kic_scale=g.get("kic_scale"),
                               qk_dtype=W.qk_dtype)
        o1, o2 = ops.hybrid_attend(
            dict(q=g["q"], kc=g["kc"], vc=g["vc"], idx=idx, pos0=pos0, max_pos=W.ctx - 1,
                 window=W.window, kw=g["kw"], vw=g["vw"], raw_pos0=rp0, sink=g["sink"]),
            dict(q=g["q_hca"], kc=g["kc_hca"], vc=g["vc_hca"], m_prime=W.m_hca, pos0=pos0,
                 max_pos=W.ctx - 1, sink=g["sink_hca"]))
        return idx, o1, o2

    ref = [t.clone() for t in step()]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for r in range(4):
        for t in outs:
            t.fill_(0)                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(_bits(got), _bits(want)), f"replay {r} differs"
        step()                              # an eager step in between
        torch.cuda.synchronize()
