"""Torch-facing wrappers over the C ABI (argument marshalling only).

Every step of the computation runs in the HIP kernels of libcsa_mi355x.so;
PyTorch only provides device memory (outputs and workspace are allocated
with torch.empty on the inputs' device) and the current HIP stream.
"""
from __future__ import annotations

import torch

from . import _lib as L

_ATTN_DT = {torch.float32: L.F32, torch.bfloat16: L.BF16}


def _p(t):
    return None if t is None else t.data_ptr()


def _dev_check(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _attn_dt(t):
    try:
        return _ATTN_DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _ws(nbytes: int, dev):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


def compress(k, v, ki, gate, m, pos_bias=None, Nc_cap=None, width=None):
    """Softmax-gated block pooling.  k, v [B,T,d]; ki [B,T,dI] or None;
    gate [d] fp32; pos_bias [width] fp32 or None; width (m..2m, default m)
    tokens pooled per entry, ending where the entry's block ends.  Returns kc,
    vc [B,Nc_cap,d], kic [B,Nc_cap,dI] (None without ki); rows >= T//m are
    left unwritten."""
    dev = _dev_check(k, v, ki, gate, pos_bias)
    B, T, d = k.shape
    dI = ki.shape[-1] if ki is not None else 0
    cap = T // m if Nc_cap is None else Nc_cap
    kc = torch.empty(B, cap, d, dtype=k.dtype, device=dev)
    vc = torch.empty_like(kc)
    kic = torch.empty(B, cap, dI, dtype=k.dtype, device=dev) if ki is not None else None
    L.check(L.load().csa_compress_window(_p(k), _p(v), _p(ki), _p(gate), _p(pos_bias), B, T, d,
                                         dI, m, m if width is None else width, cap, _attn_dt(k),
                                         _p(kc), _p(vc), _p(kic), _stream(dev)))
    return kc, vc, kic


def _qk_code(qi, qk_dtype):
    if qk_dtype is None:
        if qi.dtype == torch.float32:
            return L.F32
        if qi.dtype == torch.bfloat16:
            return L.BF16
        raise ValueError("uint8 indexer inputs need qk_dtype='fp8' or 'fp4'")
    return {"f32": L.F32, "bf16": L.BF16, "fp8": L.FP8_E4M3, "fp4": L.FP4_E2M1}[qk_dtype]


def indexer_topk(qi, w, kic, pos0, m, topk, max_pos, qi_scale=None, kic_scale=None,
                 qk_dtype=None, return_scores=False):
    """Lightning-indexer scores + lowest-index top-k.  qi [B,Tq,HI,dI] (FP4:
    [..,dI/2] packed), w [B,Tq,HI] fp32, kic [B,Nc_cap,dI] (FP4 [..,dI/2]),
    pos0 [B] int32 (positions of the first query).  Returns idx [B,Tq,topk]
    int32 (and scores [B,Tq,topk] fp32 if asked)."""
    dev = _dev_check(qi, w, kic, pos0, qi_scale, kic_scale)
    code = _qk_code(qi, qk_dtype)
    B, Tq, HI = w.shape
    dI = qi.shape[-1] * (2 if code == L.FP4_E2M1 else 1)
    Nc_cap = kic.shape[1]
    lib = L.load()
    nws = lib.csa_indexer_topk_workspace(B, Tq, Nc_cap, HI, dI, topk, code)
    ws = _ws(nws, dev)
    idx = torch.empty(B, Tq, topk, dtype=torch.int32, device=dev)
    sc = torch.empty(B, Tq, topk, dtype=torch.float32, device=dev) if return_scores else None
    L.check(lib.csa_indexer_topk(_p(qi), _p(qi_scale), _p(w), _p(kic), _p(kic_scale), _p(pos0),
                                 int(max_pos), B, Tq, Nc_cap, HI, dI, m, topk, code, _p(idx),
                                 _p(sc), _p(ws), nws, _stream(dev)))
    return (idx, sc) if return_scores else idx


def sparse_attend(q, kc, vc, idx, pos0, max_pos, window, kw=None, vw=None, raw_pos0=None,
                  sink=None, scale=None, return_lse=False):
    """CSA core attention.  q [B,Tq,H,d]; kc, vc [B,Nc_cap,d]; idx [B,Tq,k];
    kw, vw [B,R,d] raw tokens with row r at position raw_pos0[b]+r."""
    dev = _dev_check(q, kc, vc, idx, pos0, kw, vw, raw_pos0, sink)
    B, Tq, H, d = q.shape
    topk = idx.shape[-1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    lib = L.load()
    nws = lib.csa_sparse_attend_workspace(B, Tq, H, d, topk, window)
    ws = _ws(nws, dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if return_lse else None
    L.check(lib.csa_sparse_attend(_p(q), _p(kc), _p(vc), _p(idx), topk, _p(kw), _p(vw),
                                  _p(raw_pos0), R, _p(pos0), int(max_pos), window, _p(sink),
                                  float(scale), B, Tq, H, d, kc.shape[1], _attn_dt(q), _p(out),
                                  _p(lse), _p(ws), nws, _stream(dev)))
    return (out, lse) if return_lse else out


def hca_attend(q, kc, vc, m_prime, pos0, max_pos, sink=None, scale=None, window=0, kw=None,
               vw=None, raw_pos0=None, return_lse=False):
    """HCA dense attention over completed m'-blocks (+ optional window)."""
    dev = _dev_check(q, kc, vc, pos0, kw, vw, raw_pos0, sink)
    B, Tq, H, d = q.shape
    Nc_cap = kc.shape[1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    lib = L.load()
    nws = lib.hca_attend_workspace(B, Tq, H, d, Nc_cap, m_prime, window)
    ws = _ws(nws, dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if return_lse else None
    L.check(lib.hca_attend(_p(q), _p(kc), _p(vc), m_prime, Nc_cap, _p(kw), _p(vw), _p(raw_pos0),
                           R, window, _p(pos0), int(max_pos), _p(sink), float(scale), B, Tq, H, d,
                           _attn_dt(q), _p(out), _p(lse), _p(ws), nws, _stream(dev)))
    return (out, lse) if return_lse else out


def hybrid_attend(csa, hca, return_lse=False):
    """CSA and HCA attention of one layer pair in one library call.

    `csa` holds the arguments of sparse_attend (q, kc, vc, idx, pos0, max_pos,
    window, and optionally kw, vw, raw_pos0, sink, scale), `hca` those of
    hca_attend (q, kc, vc, m_prime, pos0, max_pos, and optionally sink, scale,
    window, kw, vw, raw_pos0).  Returns (csa_out, hca_out), or with return_lse
    (csa_out, csa_lse, hca_out, hca_lse)."""
    c = dict(kw=None, vw=None, raw_pos0=None, sink=None, scale=None)
    c.update(csa)
    h = dict(sink=None, scale=None, window=0, kw=None, vw=None, raw_pos0=None)
    h.update(hca)
    dev = _dev_check(c["q"], c["kc"], c["vc"], c["idx"], c["pos0"], c["kw"], c["vw"],
                     c["raw_pos0"], c["sink"], h["q"], h["kc"], h["vc"], h["pos0"], h["kw"],
                     h["vw"], h["raw_pos0"], h["sink"])
    lib = L.load()
    B, Tq, H, d = c["q"].shape
    topk = c["idx"].shape[-1]
    R = c["kw"].shape[1] if c["kw"] is not None else 0
    scale = d ** -0.5 if c["scale"] is None else c["scale"]
    nws = lib.csa_sparse_attend_workspace(B, Tq, H, d, topk, c["window"])
    ws = _ws(nws, dev)
    out = torch.empty_like(c["q"])
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if return_lse else None
    hB, hTq, hH, hd = h["q"].shape
    hNc = h["kc"].shape[1]
    hR = h["kw"].shape[1] if h["kw"] is not None else 0
    hscale = hd ** -0.5 if h["scale"] is None else h["scale"]
    hnws = lib.hca_attend_workspace(hB, hTq, hH, hd, hNc, h["m_prime"], h["window"])
    hws = _ws(hnws, dev)
    hout = torch.empty_like(h["q"])
    hlse = torch.empty(hB, hTq, hH, dtype=torch.float32, device=dev) if return_lse else None
    L.check(lib.csa_hybrid_attend(
        _p(c["q"]), _p(c["kc"]), _p(c["vc"]), _p(c["idx"]), topk, _p(c["kw"]), _p(c["vw"]),
        _p(c["raw_pos0"]), R, _p(c["pos0"]), int(c["max_pos"]), c["window"], _p(c["sink"]),
        float(scale), B, Tq, H, d, c["kc"].shape[1], _attn_dt(c["q"]), _p(out), _p(lse), _p(ws), nws,
        _p(h["q"]), _p(h["kc"]), _p(h["vc"]), h["m_prime"], hNc, _p(h["kw"]), _p(h["vw"]),
        _p(h["raw_pos0"]), hR, h["window"], _p(h["pos0"]), int(h["max_pos"]), _p(h["sink"]),
        float(hscale), hB, hTq, hH, hd, _attn_dt(h["q"]), _p(hout), _p(hlse), _p(hws), hnws,
        _stream(dev)))
    return (out, lse, hout, hlse) if return_lse else (out, hout)


def grouped_out_proj(o, w):
    """Grouped output projection.  o [T, H, d]; w [G, dg, (H/G) d] -> y [T, G dg]."""
    dev = _dev_check(o, w)
    T, H, d = o.shape
    G, dg, K = w.shape
    if K * G != H * d:
        raise ValueError("w must be [G, dg, (H/G)*d]")
    if w.dtype != o.dtype:
        raise ValueError("o and w must have the same dtype")
    y = torch.empty(T, G * dg, dtype=o.dtype, device=dev)
    lib = L.load()
    L.check(lib.csa_grouped_out_proj(_p(o), _p(w), T, H, d, G, dg, _attn_dt(o), _p(y), _stream(dev)))
    return y


def sparse_attend_kv8(q, cache, idx, pos0, max_pos, window, kw=None, vw=None, raw_pos0=None,
                      sink=None, scale=None, return_lse=False):
    """CSA core attention over FP8/BF16-RoPE caches.  cache = (k8 [B,N,d/2] uint8,
    krope [B,N,d/2] bf16, kscale [B,N] f32, v8 [B,N,d] uint8, vscale [B,N] f32);
    other arguments as sparse_attend (q, kw, vw bf16)."""
    k8, krope, ks, v8, vs = cache
    dev = _dev_check(q, k8, krope, ks, v8, vs, idx, pos0, kw, vw, raw_pos0, sink)
    B, Tq, H, d = q.shape
    topk = idx.shape[-1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    lib = L.load()
    nws = lib.csa_sparse_attend_workspace(B, Tq, H, d, topk, window)
    ws = _ws(nws, dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if return_lse else None
    L.check(lib.csa_sparse_attend_kv8(_p(q), _p(k8), _p(krope), _p(ks), _p(v8), _p(vs), _p(idx),
                                      topk, _p(kw), _p(vw), _p(raw_pos0), R, _p(pos0),
                                      int(max_pos), window, _p(sink), float(scale), B, Tq, H, d,
                                      k8.shape[1], _p(out), _p(lse), _p(ws), nws, _stream(dev)))
    return (out, lse) if return_lse else out


def hca_attend_kv8(q, cache, m_prime, pos0, max_pos, sink=None, scale=None, window=0, kw=None,
                   vw=None, raw_pos0=None, return_lse=False):
    """HCA dense attention over FP8/BF16-RoPE caches (cache as sparse_attend_kv8)."""
    k8, krope, ks, v8, vs = cache
    dev = _dev_check(q, k8, krope, ks, v8, vs, pos0, kw, vw, raw_pos0, sink)
    B, Tq, H, d = q.shape
    Nc_cap = k8.shape[1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    lib = L.load()
    nws = lib.hca_attend_workspace(B, Tq, H, d, Nc_cap, m_prime, window)
    ws = _ws(nws, dev)
    out = torch.empty_like(q)
    lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev) if return_lse else None
    L.check(lib.hca_attend_kv8(_p(q), _p(k8), _p(krope), _p(ks), _p(v8), _p(vs), m_prime, Nc_cap,
                               _p(kw), _p(vw), _p(raw_pos0), R, window, _p(pos0), int(max_pos),
                               _p(sink), float(scale), B, Tq, H, d, _p(out), _p(lse), _p(ws), nws,
                               _stream(dev)))
    return (out, lse) if return_lse else out

