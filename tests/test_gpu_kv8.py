"""GPU parity of the attention over mixed-precision caches (FP8 E4M3 codes
with a scale per row, BF16 RoPE half of the key): against the fp64 oracle on
the dequantized caches (power-of-two and general scales), and, for
power-of-two scales, bitwise against the bf16 kernels run on bf16 caches
holding the same dequantized values (scaling the fp32 partial sums by a power
of two is exact, so both kernels compute the same numbers)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, dev, f64
from oracle import formats
from sparse_attention_17_amd import ops
from synth import configs, inputs, quant

pytestmark = pytest.mark.gpu


def _dequant(k8, krope, ks, v8, vs):
    """fp64 caches from the stored codes (oracle decoder)."""
    kd = np.concatenate([formats.dequant_fp8_rows(k8.numpy(), ks.numpy()), f64(krope)], axis=-1)
    vd = formats.dequant_fp8_rows(v8.numpy(), vs.numpy())
    return kd, vd


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_csa_decode_kv8():
    w = configs.CSA_DECODE_128K.with_(ctx=4 * 6000, B=3, topk=1024)
    x = inputs.make_inputs(w, peaky=True)
    cache = quant.quant_kv8(x["kc"], x["vc"])
    kd, vd = _dequant(*cache)
    g = {k: v.to(dev()) for k, v in x.items()}
    c = tuple(t.to(dev()) for t in cache)
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev())
    idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1)
    out, lse = ops.sparse_attend_kv8(g["q"], c, idx, pos0, w.ctx - 1, w.window, kw=g["kw"],
                                     vw=g["vw"], raw_pos0=rp0, sink=g["sink"], return_lse=True)
    # the bf16 kernels on bf16 caches holding the dequantized values
    kb = torch.from_numpy(kd).to(torch.bfloat16).to(dev())
    vb = torch.from_numpy(vd).to(torch.bfloat16).to(dev())
    ref_o, ref_l = ops.sparse_attend(g["q"], kb, vb, idx, pos0, w.ctx - 1, w.window, kw=g["kw"],
                                     vw=g["vw"], raw_pos0=rp0, sink=g["sink"], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(lse, ref_l)
    idx_np = idx.cpu().numpy()
    for b in range(w.B):
        ro, rl = oracle.csa.sparse_attend(f64(x["q"][b]), kd[b], vd[b], idx_np[b], f64(x["kw"][b]),
                                          f64(x["vw"][b]), w.ctx - w.window, [w.ctx - 1], w.window,
                                          f64(x["sink"]), w.scale)
        assert_close(out[b], ro, "bf16", f"kv8 csa[{b}]", lse[b], rl)


def test_hca_decode_kv8():
    w = configs.HCA_1M_DECODE.with_(B=2, ctx=128 * 3000 + 77)
    x = inputs.make_inputs(w, peaky=True)
    cache = quant.quant_kv8(x["kc_hca"], x["vc_hca"])
    kd, vd = _dequant(*cache)
    g = {k: v.to(dev()) for k, v in x.items()}
    c = tuple(t.to(dev()) for t in cache)
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    out, lse = ops.hca_attend_kv8(g["q_hca"], c, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                  return_lse=True)
    kb = torch.from_numpy(kd).to(torch.bfloat16).to(dev())
    vb = torch.from_numpy(vd).to(torch.bfloat16).to(dev())
    ref_o, ref_l = ops.hca_attend(g["q_hca"], kb, vb, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                  return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(lse, ref_l)
    for b in range(w.B):
        ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), kd[b], vd[b], w.m_hca, [w.ctx - 1],
                                       f64(x["sink_hca"]), w.scale)
        assert_close(out[b], ro, "bf16", f"kv8 hca[{b}]", lse[b], rl)


def test_csa_prefill_kv8_with_window():
    # prefill: tiles that hold FP8 entries and bf16 window rows together
    w = configs.CSA_PREFILL_32K.with_(ctx=2048, Tq=2048)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    pos0 = torch.zeros(1, dtype=torch.int32, device=dev())
    kc, vc, kic = ops.compress(g["k"], g["v"], g["ki"], g["g"], w.m)
    idx = ops.indexer_topk(g["qi"], g["w"], kic, pos0, w.m, w.topk, max_pos=w.ctx - 1)
    cache = quant.quant_kv8(kc.cpu(), vc.cpu())
    kd, vd = _dequant(*cache)
    c = tuple(t.to(dev()) for t in cache)
    out, lse = ops.sparse_attend_kv8(g["q"], c, idx, pos0, w.ctx - 1, w.window, kw=g["k"],
                                     vw=g["v"], raw_pos0=pos0, sink=g["sink"], return_lse=True)
    kb = torch.from_numpy(kd).to(torch.bfloat16).to(dev())
    vb = torch.from_numpy(vd).to(torch.bfloat16).to(dev())
    ref_o, ref_l = ops.sparse_attend(g["q"], kb, vb, idx, pos0, w.ctx - 1, w.window, kw=g["k"],
                                     vw=g["v"], raw_pos0=pos0, sink=g["sink"], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(lse, ref_l)
    ts = np.r_[0:3, 700:703, 2045:2048]
    idx_np = idx.cpu().numpy()
    ro, rl = oracle.csa.sparse_attend(f64(x["q"][0, ts]), kd[0], vd[0], idx_np[0, ts], f64(x["k"][0]),
                                      f64(x["v"][0]), 0, ts, w.window, f64(x["sink"]), w.scale)
    assert_close(out[0, ts], ro, "bf16", "kv8 prefill", lse[0, ts], rl)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_decode_kv8_general_scales(kind):
    # row scales that are not powers of two (amax / 448): the codes are widened
    # exactly and the scales multiply the fp32 logits of the code half and the
    # probabilities, so even the sharp ("peaky": q x 4d) softmax stays within
    # the bf16 output and lse tolerances against the oracle on code x scale
    if kind == "csa":
        w = configs.CSA_DECODE_128K.with_(ctx=4 * 6000, B=2, topk=1024)
        x = inputs.make_inputs(w, peaky=True)
        kc, vc = x["kc"], x["vc"]
    else:
        w = configs.HCA_1M_DECODE.with_(B=2, ctx=128 * 1500)
        x = inputs.make_inputs(w, peaky=True)
        kc, vc = x["kc_hca"], x["vc_hca"]
    k8, ks = quant.quant_fp8_rows(kc[..., :64].float())
    v8, vs = quant.quant_fp8_rows(vc.float())
    krope = kc[..., 64:].contiguous()
    assert not torch.all(torch.frexp(ks)[0] == 0.5)          # some scale is not a power of two
    kd, vd = _dequant(k8, krope, ks, v8, vs)
    g = {k: v.to(dev()) for k, v in x.items()}
    c = tuple(t.to(dev()) for t in (k8, krope, ks, v8, vs))
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    if kind == "csa":
        rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev())
        idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1)
        out, lse = ops.sparse_attend_kv8(g["q"], c, idx, pos0, w.ctx - 1, w.window, kw=g["kw"],
                                         vw=g["vw"], raw_pos0=rp0, sink=g["sink"], return_lse=True)
        idx_np = idx.cpu().numpy()
    else:
        out, lse = ops.hca_attend_kv8(g["q_hca"], c, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                      return_lse=True)
    torch.cuda.synchronize()
    for b in range(w.B):
        if kind == "csa":
            ro, rl = oracle.csa.sparse_attend(f64(x["q"][b]), kd[b], vd[b], idx_np[b], f64(x["kw"][b]),
                                              f64(x["vw"][b]), w.ctx - w.window, [w.ctx - 1],
                                              w.window, f64(x["sink"]), w.scale)
        else:
            ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), kd[b], vd[b], w.m_hca, [w.ctx - 1],
                                           f64(x["sink_hca"]), w.scale)
        assert_close(out[b], ro, "bf16", f"kv8 {kind} general scales [{b}]", lse[b], rl)


@pytest.mark.parametrize("H,Tq", [(16, 1), (48, 40), (64, 70), (128, 1)])
def test_hca_kv8_other_tile_shapes(H, Tq):
    # query tiles of 16, 96, 128 and 128 rows: the other wave layouts of the kernel
    w = configs.HCA_1M_DECODE.with_(B=2, H=H, Tq=Tq, ctx=128 * 700 + 5)
    x = inputs.make_inputs(w)
    cache = quant.quant_kv8(x["kc_hca"], x["vc_hca"])
    kd, vd = _dequant(*cache)
    g = {k: v.to(dev()) for k, v in x.items()}
    c = tuple(t.to(dev()) for t in cache)
    pos0 = torch.full((w.B,), w.ctx - Tq, dtype=torch.int32, device=dev())
    out, lse = ops.hca_attend_kv8(g["q_hca"], c, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                  return_lse=True)
    kb = torch.from_numpy(kd).to(torch.bfloat16).to(dev())
    vb = torch.from_numpy(vd).to(torch.bfloat16).to(dev())
    ref_o, ref_l = ops.hca_attend(g["q_hca"], kb, vb, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                  return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(lse, ref_l)
    pos = np.arange(w.ctx - Tq, w.ctx)
    for b in range(w.B):
        ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), kd[b], vd[b], w.m_hca, pos,
                                       f64(x["sink_hca"]), w.scale)
        assert_close(out[b], ro, "bf16", f"kv8 hca H={H} Tq={Tq} [{b}]", lse[b], rl)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_kv8_shared_entry(kind):
    # values are the key rows themselves (v8 = vscale = NULL)
    if kind == "csa":
        w = configs.CSA_DECODE_128K.with_(ctx=4 * 6000, B=2, topk=1024)
        x = inputs.make_inputs(w, peaky=True)
        kc = x["kc"]
    else:
        w = configs.HCA_1M_DECODE.with_(B=2, ctx=128 * 3000 + 77)
        x = inputs.make_inputs(w, peaky=True)
        kc = x["kc_hca"]
    k8, krope, ks, _, _ = quant.quant_kv8(kc, kc)
    kd = np.concatenate([formats.dequant_fp8_rows(k8.numpy(), ks.numpy()), f64(krope)], axis=-1)
    g = {k: v.to(dev()) for k, v in x.items()}
    c = (k8.to(dev()), krope.to(dev()), ks.to(dev()), None, None)
    kb = torch.from_numpy(kd).to(torch.bfloat16).to(dev())
    pos0 = torch.full((w.B,), w.ctx - 1, dtype=torch.int32, device=dev())
    if kind == "csa":
        rp0 = torch.full((w.B,), w.ctx - w.window, dtype=torch.int32, device=dev())
        idx = ops.indexer_topk(g["qi"], g["w"], g["kic"], pos0, w.m, w.topk, max_pos=w.ctx - 1)
        out, lse = ops.sparse_attend_kv8(g["q"], c, idx, pos0, w.ctx - 1, w.window, kw=g["kw"],
                                         vw=g["vw"], raw_pos0=rp0, sink=g["sink"], return_lse=True)
        ref_o, ref_l = ops.sparse_attend(g["q"], kb, kb, idx, pos0, w.ctx - 1, w.window, kw=g["kw"],
                                         vw=g["vw"], raw_pos0=rp0, sink=g["sink"], return_lse=True)
    else:
        out, lse = ops.hca_attend_kv8(g["q_hca"], c, w.m_hca, pos0, w.ctx - 1, sink=g["sink_hca"],
                                      return_lse=True)
        ref_o, ref_l = ops.hca_attend(g["q_hca"], kb, kb, w.m_hca, pos0, w.ctx - 1,
                                      sink=g["sink_hca"], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref_o)) and torch.equal(lse, ref_l)
    for b in range(w.B):
        if kind == "csa":
            ro, rl = oracle.csa.sparse_attend(f64(x["q"][b]), kd[b], kd[b], idx.cpu().numpy()[b],
                                              f64(x["kw"][b]), f64(x["vw"][b]), w.ctx - w.window,
                                              [w.ctx - 1], w.window, f64(x["sink"]), w.scale)
        else:
            ro, rl = oracle.hca.hca_attend(f64(x["q_hca"][b]), kd[b], kd[b], w.m_hca, [w.ctx - 1],
                                           f64(x["sink_hca"]), w.scale)
        assert_close(out[b], ro, "bf16", f"kv8 shared {kind}[{b}]", lse[b], rl)
