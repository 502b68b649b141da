"""Seeded synthetic tensors for a workload.

Every tensor is drawn as standard normal fp32 from
numpy.random.default_rng(SeedSequence([seed, workload id, tensor id])),
scaled by 1/sqrt(its last dim) for q, k, v, indexer q/k and caches (gates,
sinks and head-weight logits stay unscaled N(0,1)), then rounded to the
workload's storage dtype (bf16 with round-to-nearest-even) or encoded to
FP8/FP4 codes.  Tensors are returned as CPU torch tensors; callers move them
to the device or widen them to float64 for the oracle.

"peaky" multiplies the attention queries by 4*d and the sink logits by 4, so
that softmax-scaled logits have std ~4 and attention selects sharply.
"""
from __future__ import annotations

import numpy as np
import torch

from . import quant
from .configs import Workload

SEED = 17
TID = dict(q=0, k=1, v=2, ki=3, qi=4, wlog=5, g=6, g_hca=7, sink=8, kic=9, kc=10, vc=11,
           kw=12, vw=13, q_hca=14, kc_hca=15, vc_hca=16, sink_hca=17, pos_bias=18,
           pos_bias_hca=19, o_attn=20, w_proj=21)


def rng_for(wid: int, tensor: str, seed: int = SEED) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, wid, TID[tensor]]))


def normal(wid: int, tensor: str, shape, scaled_by_last: bool = True, seed: int = SEED):
    a = rng_for(wid, tensor, seed).standard_normal(shape, dtype=np.float32)
    if scaled_by_last:
        a *= np.float32(1.0 / np.sqrt(shape[-1]))
    return torch.from_numpy(a)


def to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.float().contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def make_inputs(w: Workload, seed: int = SEED, peaky: bool = False,
                pos_bias: bool = False) -> dict:
    """Returns a dict of CPU tensors.  Keys present depend on the workload:

    prefill (raw tokens given): k, v [B,ctx,d]; ki [B,ctx,dI]; g [d]; g_hca [d]
    decode (caches given):      kc, vc [B,Nc,d]; kic (bf16/f32 [B,Nc,dI], or
                                codes + kic_scale); kw, vw [B,window,d]
    HCA decode:                 kc_hca, vc_hca [B,Nc_hca,d]
    always: q [B,Tq,H,d] (CSA), q_hca (HCA), qi / qi_scale, w [B,Tq,HI]
    (softmax over the indexer heads of seeded logits), sink / sink_hca [H].
    """
    out = {}
    B, H, d, Tq, wid = w.B, w.H, w.d, w.Tq, w.wid
    dt = w.dtype
    qmul = float(4 * d) if peaky else 1.0
    smul = 4.0 if peaky else 1.0

    if w.mode == "prefill":
        out["k"] = to_dtype(normal(wid, "k", (B, w.ctx, d), seed=seed), dt)
        out["v"] = to_dtype(normal(wid, "v", (B, w.ctx, d), seed=seed), dt)
        if w.has_csa:
            out["ki"] = to_dtype(normal(wid, "ki", (B, w.ctx, w.dI), seed=seed), dt)
            out["g"] = normal(wid, "g", (d,), False, seed=seed)
            if pos_bias:
                out["pos_bias"] = normal(wid, "pos_bias", (w.m,), False, seed=seed)
        if w.has_hca:
            out["g_hca"] = normal(wid, "g_hca", (d,), False, seed=seed)
            if pos_bias:
                out["pos_bias_hca"] = normal(wid, "pos_bias_hca", (w.m_hca,), False, seed=seed)
    else:
        if w.has_csa:
            out["kc"] = to_dtype(normal(wid, "kc", (B, w.Nc, d), seed=seed), dt)
            out["vc"] = to_dtype(normal(wid, "vc", (B, w.Nc, d), seed=seed), dt)
            out["kw"] = to_dtype(normal(wid, "kw", (B, w.window, d), seed=seed), dt)
            out["vw"] = to_dtype(normal(wid, "vw", (B, w.window, d), seed=seed), dt)
            kic = normal(wid, "kic", (B, w.Nc, w.dI), seed=seed)
            _encode_qk(out, "kic", kic, w.qk_dtype, dt)
        if w.has_hca:
            out["kc_hca"] = to_dtype(normal(wid, "kc_hca", (B, w.Nc_hca, d), seed=seed), dt)
            out["vc_hca"] = to_dtype(normal(wid, "vc_hca", (B, w.Nc_hca, d), seed=seed), dt)

    if w.has_csa:
        q = normal(wid, "q", (B, Tq, H, d), seed=seed) * qmul
        out["q"] = to_dtype(q, dt)
        qi = normal(wid, "qi", (B, Tq, w.HI, w.dI), seed=seed)
        _encode_qk(out, "qi", qi, w.qk_dtype, dt)
        wl = normal(wid, "wlog", (B, Tq, w.HI), False, seed=seed)
        out["w"] = torch.softmax(wl.double(), dim=-1).float().contiguous()
        out["sink"] = normal(wid, "sink", (H,), False, seed=seed) * smul
    if w.has_hca:
        qh = normal(wid, "q_hca", (B, Tq, H, d), seed=seed) * qmul
        out["q_hca"] = to_dtype(qh, dt)
        out["sink_hca"] = normal(wid, "sink_hca", (H,), False, seed=seed) * smul
    return out


def _encode_qk(out: dict, name: str, x: torch.Tensor, qk_dtype: str, dt: str) -> None:
    if qk_dtype in ("f32", "bf16"):
        out[name] = to_dtype(x, qk_dtype)
    elif qk_dtype == "fp8":
        out[name], out[name + "_scale"] = quant.quant_fp8_rows(x)
    elif qk_dtype == "fp4":
        out[name], out[name + "_scale"] = quant.quant_fp4_blocks(x)
    else:
        raise ValueError(qk_dtype)


def proj_inputs(wid: int, T: int, H: int, d: int, G: int, dg: int, dtype: str, seed: int = SEED):
    """Attention outputs o [T, H, d] ~ N(0, 1) and group weights w [G, dg, (H/G) d]
    ~ N(0, 1/((H/G) d)) for the grouped output projection (values, no method
    arithmetic), in the given dtype."""
    o = normal(wid, "o_attn", (T, H, d), scaled_by_last=False, seed=seed)
    w = normal(wid, "w_proj", (G, dg, (H // G) * d), scaled_by_last=False, seed=seed)
    w *= np.float32(1.0 / np.sqrt((H // G) * d))
    return to_dtype(o, dtype), to_dtype(w, dtype)

