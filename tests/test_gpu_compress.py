"""GPU parity of csa_compress against the fp64 oracle: fp32 within 1e-5
max-abs, bf16 within one bf16 ulp of the exact pooled value; overlapping
windows (csa_compress_window) within the fp32 / bf16 output tolerances."""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, bf16_ulp_ok, dev, f64, pool_slack
from sparse_attention_17_amd import ops
from synth import configs, inputs

pytestmark = pytest.mark.gpu


def _run(x, gate_key, m, with_ki, pos_bias=None, cap=None):
    g = {k: v.to(dev()) for k, v in x.items()}
    pb = g.get(pos_bias) if pos_bias else None
    kc, vc, kic = ops.compress(g["k"], g["v"], g["ki"] if with_ki else None, g[gate_key], m,
                               pos_bias=pb, Nc_cap=cap)
    torch.cuda.synchronize()
    return kc, vc, kic


def _oracle(x, gate_key, m, b, with_ki, pos_bias=None):
    return oracle.csa.compress(f64(x["k"][b]), f64(x["v"][b]), f64(x["ki"][b]) if with_ki else None,
                               f64(x[gate_key]), m, None if pos_bias is None else f64(x[pos_bias]))


@pytest.mark.parametrize("pb", [False, True])
def test_tiny_f32_csa_and_hca(pb):
    w = configs.TINY
    x = inputs.make_inputs(w, pos_bias=True)
    for gate, m, ki, pbk in (("g", w.m, True, "pos_bias"), ("g_hca", w.m_hca, False, "pos_bias_hca")):
        kc, vc, kic = _run(x, gate, m, ki, pbk if pb else None)
        rk, rv, rki = _oracle(x, gate, m, 0, ki, pbk if pb else None)
        assert_close(kc[0], rk, "f32", "kc")
        assert_close(vc[0], rv, "f32", "vc")
        if ki:
            assert_close(kic[0], rki, "f32", "kic")


@pytest.mark.parametrize("T,m,d,dI,B", [(4096, 4, 128, 64, 2), (16384, 128, 128, 64, 1),
                                        (1030, 4, 64, 32, 3), (640, 5, 128, 32, 1),
                                        (256, 1, 64, 64, 1)])
def test_bf16_within_one_ulp(T, m, d, dI, B):
    w = configs.CSA_PREFILL_32K.with_(ctx=T, Tq=T, d=d, dI=dI, m=m, B=B)
    x = inputs.make_inputs(w, pos_bias=True)
    kc, vc, kic = _run(x, "g", m, True, "pos_bias")
    for b in range(B):
        rk, rv, rki = _oracle(x, "g", m, b, True, "pos_bias")
        for got, ref, nm, src in ((kc[b], rk, "kc", "k"), (vc[b], rv, "vc", "v"),
                                  (kic[b], rki, "kic", "ki")):
            nbad, worst = bf16_ulp_ok(got, ref, 1.0, pool_slack(f64(x[src][b]), m))
            assert nbad == 0, f"{nm}[{b}]: {nbad} values beyond 1 ulp (worst {worst:.2f} ulp)"
    if m == 1:   # pooling one token is the identity, exactly
        assert torch.equal(kc.cpu(), x["k"]) and torch.equal(vc.cpu(), x["v"])


def test_rows_beyond_T_over_m_untouched():
    w = configs.TINY.with_(ctx=1030, Tq=1030)
    x = inputs.make_inputs(w)
    g = {k: v.to(dev()) for k, v in x.items()}
    cap = 300
    from sparse_attention_17_amd import _lib as L
    kc = torch.full((1, cap, 64), 7.0, device=dev())
    vc = torch.full((1, cap, 64), 7.0, device=dev())
    L.check(L.load().csa_compress(g["k"].data_ptr(), g["v"].data_ptr(), None, g["g"].data_ptr(),
                                  None, 1, 1030, 64, 32, 4, cap, L.F32, kc.data_ptr(),
                                  vc.data_ptr(), None, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert torch.all(kc[0, 257:] == 7.0) and torch.all(vc[0, 257:] == 7.0)
    rk, rv, _ = _oracle(x, "g", 4, 0, False)
    assert_close(kc[0, :257], rk, "f32", "kc")


def test_hca_1m_compress_sample():
    # m'=128 over 1M tokens (one sequence): checks sampled blocks
    w = configs.CSA_PREFILL_32K.with_(ctx=1 << 20, Tq=1, m=128, dI=64, B=1)
    k = inputs.to_dtype(inputs.normal(40, "k", (1, 1 << 20, 128)), "bf16")
    v = inputs.to_dtype(inputs.normal(40, "v", (1, 1 << 20, 128)), "bf16")
    gate = inputs.normal(40, "g_hca", (128,), False)
    kc, vc, _ = ops.compress(k.to(dev()), v.to(dev()), None, gate.to(dev()), 128)
    torch.cuda.synchronize()
    assert kc.shape == (1, 8192, 128)
    blocks = np.r_[0:4, 4096:4100, 8188:8192]
    for j in blocks:
        sl = slice(j * 128, (j + 1) * 128)
        rk, rv, _ = oracle.csa.compress(f64(k[0, sl]), f64(v[0, sl]), None, f64(gate), 128)
        assert bf16_ulp_ok(kc[0, j], rk[0], 1.0, pool_slack(f64(k[0, sl]), 128)[0])[0] == 0
        assert bf16_ulp_ok(vc[0, j], rv[0], 1.0, pool_slack(f64(v[0, sl]), 128)[0])[0] == 0
    del w


@pytest.mark.parametrize("dtype,T,m,width,B", [("f32", 1024, 4, 8, 1), ("f32", 1030, 4, 5, 2),
                                               ("bf16", 32768, 4, 8, 1), ("bf16", 4099, 5, 10, 2),
                                               ("bf16", 2048, 128, 256, 1)])
def test_overlapping_windows(dtype, T, m, width, B):
    # each entry pools the `width` tokens ending at its block's end (csa_compress_window)
    base = configs.TINY if dtype == "f32" else configs.CSA_PREFILL_32K
    w = base.with_(ctx=T, Tq=T, m=m, B=B)
    x = inputs.make_inputs(w)
    pb = inputs.normal(w.wid, "pos_bias", (width,), False)
    g = {k: v.to(dev()) for k, v in x.items()}
    kc, vc, kic = ops.compress(g["k"], g["v"], g["ki"], g["g"], m, pos_bias=pb.to(dev()), width=width)
    torch.cuda.synchronize()
    assert kc.shape[1] == T // m
    for b in range(B):
        rk, rv, rki = oracle.csa.compress_window(f64(x["k"][b]), f64(x["v"][b]), f64(x["ki"][b]),
                                                 f64(x["g"]), m, width, f64(pb))
        assert_close(kc[b], rk, dtype, f"kc[{b}]")
        assert_close(vc[b], rv, dtype, f"vc[{b}]")
        assert_close(kic[b], rki, dtype, f"kic[{b}]")
