"""csa_hybrid_decode_step_static (scratch in the library's static per-device
array, no workspace argument) against csa_hybrid_decode_step with a caller
workspace: bitwise equal outputs on two calls in a row, the second on a
smaller step (the array keeps the first call's contents)."""
import pytest
import torch

from sparse_attention_17_amd import ops
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _step(w):
    dev = torch.device("cuda:0")
    x = inputs.make_inputs(w, peaky=True)
    g = {k: v.to(dev) for k, v in x.items()}
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev)
    rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev)
    idx = dict(qi=g["qi"], w=g["w"], kic=g["kic"], m=w.m, topk=w.topk, qi_scale=g.get("qi_scale"),
               kic_scale=g.get("kic_scale"), qk_dtype=w.qk_dtype)
    csa = dict(q=g["q"], kc=g["kc"], vc=g["vc"], window=w.window, kw=g["kw"], vw=g["vw"],
               raw_pos0=rp0, sink=g["sink"])
    hca = dict(q=g["q_hca"], kc=g["kc_hca"], vc=g["vc_hca"], m_prime=w.m_hca, sink=g["sink_hca"])
    return ops.DecodeStep(idx, csa, hca, pos0, w.ctx - 1, return_lse=True), g


def test_static_step_matches_workspace_step_twice():
    # B=8, a smaller B=3 step, then B=8 again: the static array's control words
    # must be zero for every batch size after any earlier call
    small = configs.HYBRID_1M_FP8.with_(B=3, ctx=4 * 20000 + 1, qk_dtype="bf16")
    for w in (configs.HYBRID_1M_FP8, small, configs.HYBRID_1M_FP8):
        st, _ = _step(w)
        st.run()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (st.idx, st.out, st.lse, st.hout, st.hlse)]
        for t in (st.idx, st.out, st.lse, st.hout, st.hlse):
            t.fill_(0)
        st.run_static()
        torch.cuda.synchronize()
        for a, b, nm in zip((st.idx, st.out, st.lse, st.hout, st.hlse), ref,
                            ("idx", "out", "lse", "hout", "hlse")):
            assert torch.equal(_bits(a), _bits(b)), f"B={w.B} ctx={w.ctx}: {nm} differs"
