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


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_i32(name, t, shape):
    _need(t.dtype == torch.int32, f"{name} must be int32 (got {t.dtype})")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _check_f32(name, t, shape):
    if t is None:
        return
    _need(t.dtype == torch.float32, f"{name} must be float32 (got {t.dtype})")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _check_rows(name, t, dtype, lead, d):
    """t must be [*lead, d] of `dtype`."""
    _need(t.dtype == dtype, f"{name} must be {dtype} (got {t.dtype})")
    _need(t.dim() == len(lead) + 1 and tuple(t.shape[:-1]) == tuple(lead) and t.shape[-1] == d,
          f"{name} must have shape {tuple(lead) + (d,)} (got {tuple(t.shape)})")


def _check_attend(q, kc, vc, pos0, kw, vw, raw_pos0, sink, window):
    """Shapes and dtypes shared by the attention wrappers (q [B,Tq,H,d] sets them)."""
    _need(q.dim() == 4, f"q must be [B, Tq, H, d] (got {tuple(q.shape)})")
    B, Tq, H, d = q.shape
    _need(kc.dim() == 3 and kc.shape[0] == B, f"kc must be [B={B}, Nc_cap, d] (got {tuple(kc.shape)})")
    _check_rows("kc", kc, q.dtype, (B, kc.shape[1]), d)
    if vc is not None:
        _check_rows("vc", vc, q.dtype, (B, kc.shape[1]), d)
    _check_i32("pos0", pos0, (B,))
    _check_f32("sink", sink, (H,))
    if window > 0:
        _need(kw is not None and vw is not None and raw_pos0 is not None,
              "window > 0 needs kw, vw and raw_pos0")
    if kw is not None:
        _need(kw.dim() == 3, f"kw must be [B, R, d] (got {tuple(kw.shape)})")
        _check_rows("kw", kw, q.dtype, (B, kw.shape[1]), d)
        _need(vw is not None, "kw needs vw")
        _check_rows("vw", vw, q.dtype, (B, kw.shape[1]), d)
    if raw_pos0 is not None:
        _check_i32("raw_pos0", raw_pos0, (B,))
    return B, Tq, H, d


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
    _need(k.dim() == 3, f"k must be [B, T, d] (got {tuple(k.shape)})")
    B, T, d = k.shape
    _check_rows("v", v, k.dtype, (B, T), d)
    dI = ki.shape[-1] if ki is not None else 0
    if ki is not None:
        _check_rows("ki", ki, k.dtype, (B, T), dI)
    _check_f32("gate", gate, (d,))
    _check_f32("pos_bias", pos_bias, (m if width is None else width,))
    dev = _dev_check(k, v, ki, gate, pos_bias)
    cap = T // m if Nc_cap is None else Nc_cap
    kc = torch.empty(B, cap, d, dtype=k.dtype, device=dev)
    vc = torch.empty_like(kc)
    kic = torch.empty(B, cap, dI, dtype=k.dtype, device=dev) if ki is not None else None
    lib = L.load()
    if width is None:
        L.check(lib.csa_compress(_p(k), _p(v), _p(ki), _p(gate), _p(pos_bias), B, T, d, dI, m,
                                 cap, _attn_dt(k), _p(kc), _p(vc), _p(kic), _stream(dev)))
    else:
        L.check(lib.csa_compress_window(_p(k), _p(v), _p(ki), _p(gate), _p(pos_bias), B, T, d,
                                        dI, m, width, cap, _attn_dt(k), _p(kc), _p(vc), _p(kic),
                                        _stream(dev)))
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
    code = _qk_code(qi, qk_dtype)
    _need(w.dim() == 3, f"w must be [B, Tq, HI] (got {tuple(w.shape)})")
    B, Tq, HI = w.shape
    _check_f32("w", w, (B, Tq, HI))
    dI = qi.shape[-1] * (2 if code == L.FP4_E2M1 else 1)
    _need(kic.dim() == 3 and kic.shape[0] == B, f"kic must be [B={B}, Nc_cap, ...] (got {tuple(kic.shape)})")
    Nc_cap = kic.shape[1]
    store = {L.F32: torch.float32, L.BF16: torch.bfloat16, L.FP8_E4M3: torch.uint8,
             L.FP4_E2M1: torch.uint8}[code]
    row = qi.shape[-1]
    _check_rows("qi", qi, store, (B, Tq, HI), row)
    _check_rows("kic", kic, store, (B, Nc_cap), row)
    _check_i32("pos0", pos0, (B,))
    if code == L.FP8_E4M3:
        _need(qi_scale is not None and kic_scale is not None, "FP8 needs qi_scale and kic_scale")
        _check_f32("qi_scale", qi_scale, (B, Tq, HI))
        _check_f32("kic_scale", kic_scale, (B, Nc_cap))
    elif code == L.FP4_E2M1:
        _need(qi_scale is not None and kic_scale is not None, "FP4 needs qi_scale and kic_scale")
        _check_rows("qi_scale", qi_scale, torch.uint8, (B, Tq, HI), dI // 32)
        _check_rows("kic_scale", kic_scale, torch.uint8, (B, Nc_cap), dI // 32)
    else:
        _need(qi_scale is None and kic_scale is None, "f32/bf16 indexer inputs take no scales")
    dev = _dev_check(qi, w, kic, pos0, qi_scale, kic_scale)
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
    B, Tq, H, d = _check_attend(q, kc, vc, pos0, kw, vw, raw_pos0, sink, window)
    _need(idx.dim() == 3, f"idx must be [B, Tq, topk] (got {tuple(idx.shape)})")
    topk = idx.shape[-1]
    _check_i32("idx", idx, (B, Tq, topk))
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    dev = _dev_check(q, kc, vc, idx, pos0, kw, vw, raw_pos0, sink)
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
    B, Tq, H, d = _check_attend(q, kc, vc, pos0, kw, vw, raw_pos0, sink, window)
    Nc_cap = kc.shape[1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    dev = _dev_check(q, kc, vc, pos0, kw, vw, raw_pos0, sink)
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
    B, Tq, H, d = _check_attend(c["q"], c["kc"], c["vc"], c["pos0"], c["kw"], c["vw"],
                                c["raw_pos0"], c["sink"], c["window"])
    _check_attend(h["q"], h["kc"], h["vc"], h["pos0"], h["kw"], h["vw"], h["raw_pos0"], h["sink"],
                  h["window"])
    _need(c["idx"].dim() == 3, "idx must be [B, Tq, topk]")
    _check_i32("idx", c["idx"], (B, Tq, c["idx"].shape[-1]))
    dev = _dev_check(c["q"], c["kc"], c["vc"], c["idx"], c["pos0"], c["kw"], c["vw"],
                     c["raw_pos0"], c["sink"], h["q"], h["kc"], h["vc"], h["pos0"], h["kw"],
                     h["vw"], h["raw_pos0"], h["sink"])
    lib = L.load()
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
    T, H, d = o.shape
    G, dg, K = w.shape
    if K * G != H * d:
        raise ValueError("w must be [G, dg, (H/G)*d]")
    if w.dtype != o.dtype:
        raise ValueError("o and w must have the same dtype")
    dev = _dev_check(o, w)
    y = torch.empty(T, G * dg, dtype=o.dtype, device=dev)
    lib = L.load()
    L.check(lib.csa_grouped_out_proj(_p(o), _p(w), T, H, d, G, dg, _attn_dt(o), _p(y), _stream(dev)))
    return y


def _check_kv8(q, cache, pos0, kw, vw, raw_pos0, sink, window):
    """The five planes of a mixed-precision cache against q [B,Tq,H,d] (bf16)."""
    k8, krope, ks, v8, vs = cache
    _need(q.dim() == 4 and q.dtype == torch.bfloat16, "q must be bf16 [B, Tq, H, d]")
    B, Tq, H, d = q.shape
    _need(k8.dim() == 3, f"k8 must be [B, N, d/2] (got {tuple(k8.shape)})")
    N = k8.shape[1]
    _check_rows("k8", k8, torch.uint8, (B, N), d // 2)
    _check_rows("krope", krope, torch.bfloat16, (B, N), d - d // 2)
    _check_f32("kscale", ks, (B, N))
    _need((v8 is None) == (vs is None), "v8 and vscale must both be given or both be None")
    if v8 is not None:
        _check_rows("v8", v8, torch.uint8, (B, N), d)
        _check_f32("vscale", vs, (B, N))
    _check_i32("pos0", pos0, (B,))
    _check_f32("sink", sink, (H,))
    if window > 0:
        _need(kw is not None and vw is not None and raw_pos0 is not None,
              "window > 0 needs kw, vw and raw_pos0")
    if kw is not None:
        _check_rows("kw", kw, q.dtype, (B, kw.shape[1]), d)
        _check_rows("vw", vw, q.dtype, (B, kw.shape[1]), d)
    if raw_pos0 is not None:
        _check_i32("raw_pos0", raw_pos0, (B,))
    return B, Tq, H, d


def sparse_attend_kv8(q, cache, idx, pos0, max_pos, window, kw=None, vw=None, raw_pos0=None,
                      sink=None, scale=None, return_lse=False):
    """CSA core attention over FP8/BF16-RoPE caches.  cache = (k8 [B,N,d/2] uint8,
    krope [B,N,d/2] bf16, kscale [B,N] f32, v8 [B,N,d] uint8, vscale [B,N] f32);
    other arguments as sparse_attend (q, kw, vw bf16)."""
    k8, krope, ks, v8, vs = cache
    B, Tq, H, d = _check_kv8(q, cache, pos0, kw, vw, raw_pos0, sink, window)
    _need(idx.dim() == 3, "idx must be [B, Tq, topk]")
    topk = idx.shape[-1]
    _check_i32("idx", idx, (B, Tq, topk))
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    dev = _dev_check(q, k8, krope, ks, v8, vs, idx, pos0, kw, vw, raw_pos0, sink)
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
    B, Tq, H, d = _check_kv8(q, cache, pos0, kw, vw, raw_pos0, sink, window)
    Nc_cap = k8.shape[1]
    R = kw.shape[1] if kw is not None else 0
    scale = d ** -0.5 if scale is None else scale
    dev = _dev_check(q, k8, krope, ks, v8, vs, pos0, kw, vw, raw_pos0, sink)
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


def profile_counter(name: str, reset: bool = False) -> int:
    """A device event counter of the library (csa_profile_counter): e.g.
    "indexer_prefill_fallback" counts prefill rows whose top-k took the exact
    fallback select."""
    import ctypes as C
    v = C.c_ulonglong(0)
    st = L.load().csa_profile_counter(name.encode(), C.byref(v), 1 if reset else 0)
    if st != 0:
        raise RuntimeError(f"csa_profile_counter({name!r}) returned {st}")
    return int(v.value)


class DecodeStep:
    """One decode step of a hybrid CSA + HCA layer pair (csa_hybrid_decode_step):
    the indexer and its top-k, the CSA attention and the HCA attention in one
    library call.

    Built once for a set of input tensors (validated, outputs and workspace
    allocated here, the C descriptor filled in); run() then enqueues the whole
    step with one call on the current stream.  `idx` holds the CSA index lists
    arguments as indexer_topk (qi, w, kic, m, topk, and optionally qi_scale,
    kic_scale, qk_dtype), `csa` those of sparse_attend (q, kc, vc, window, and
    optionally kw, vw, raw_pos0, sink, scale), `hca` those of hca_attend (q, kc,
    vc, m_prime, and optionally sink, scale, window, kw, vw, raw_pos0); pos0 and
    max_pos are shared.  Outputs: self.idx, self.out, self.hout (+ self.lse,
    self.hlse with return_lse).  fused_tail=True runs both attention problems
    and their merges in one kernel ordered by device counters (same
    results)."""

    def __init__(self, idx, csa, hca, pos0, max_pos, return_lse=False, fused_tail=False):
        i = dict(qi_scale=None, kic_scale=None, qk_dtype=None)
        i.update(idx)
        c = dict(kw=None, vw=None, raw_pos0=None, sink=None, scale=None)
        c.update(csa)
        h = dict(sink=None, scale=None, window=0, kw=None, vw=None, raw_pos0=None)
        h.update(hca)
        q = c["q"]
        B, Tq, H, d = _check_attend(q, c["kc"], c["vc"], pos0, c["kw"], c["vw"], c["raw_pos0"],
                                    c["sink"], c["window"])
        _need(Tq == 1, "a decode step has one query token per sequence")
        _check_attend(h["q"], h["kc"], h["vc"], pos0, h["kw"], h["vw"], h["raw_pos0"], h["sink"],
                      h["window"])
        _need(tuple(h["q"].shape) == tuple(q.shape) and h["q"].dtype == q.dtype,
              "the HCA query must have the CSA query's shape and dtype")
        code = _qk_code(i["qi"], i["qk_dtype"])
        w = i["w"]
        _check_f32("w", w, (B, 1, w.shape[-1]))
        HI = w.shape[-1]
        dI = i["qi"].shape[-1] * (2 if code == L.FP4_E2M1 else 1)
        Nc_cap = c["kc"].shape[1]
        _need(i["kic"].dim() == 3 and i["kic"].shape[:2] == (B, Nc_cap),
              f"kic must be [B, Nc_cap={Nc_cap}, ...] (the rows of kc)")
        dev = _dev_check(q, c["kc"], c["vc"], pos0, c["kw"], c["vw"], c["raw_pos0"], c["sink"],
                         h["q"], h["kc"], h["vc"], h["kw"], h["vw"], h["raw_pos0"], h["sink"],
                         i["qi"], i["qi_scale"], w, i["kic"], i["kic_scale"])
        self.idx = torch.empty(B, 1, i["topk"], dtype=torch.int32, device=dev)
        self.out = torch.empty_like(q)
        self.hout = torch.empty_like(h["q"])
        self.lse = torch.empty(B, 1, H, dtype=torch.float32, device=dev) if return_lse else None
        self.hlse = torch.empty(B, 1, H, dtype=torch.float32, device=dev) if return_lse else None
        s = L.DecodeStepDesc()
        s.B, s.pos0, s.max_pos, s.H, s.d, s.dt = B, _p(pos0), int(max_pos), H, d, _attn_dt(q)
        s.qi, s.qi_scale, s.w, s.kic, s.kic_scale = (_p(i["qi"]), _p(i["qi_scale"]), _p(w),
                                                     _p(i["kic"]), _p(i["kic_scale"]))
        s.HI, s.dI, s.m, s.topk, s.qk_dt, s.idx_out = HI, dI, i["m"], i["topk"], code, _p(self.idx)
        s.q, s.kc, s.vc, s.Nc_cap = _p(q), _p(c["kc"]), _p(c["vc"]), Nc_cap
        s.kw, s.vw, s.raw_pos0 = _p(c["kw"]), _p(c["vw"]), _p(c["raw_pos0"])
        s.R = c["kw"].shape[1] if c["kw"] is not None else 0
        s.window, s.sink = c["window"], _p(c["sink"])
        s.softmax_scale = d ** -0.5 if c["scale"] is None else c["scale"]
        s.out, s.lse_out = _p(self.out), _p(self.lse)
        s.hq, s.hkc, s.hvc = _p(h["q"]), _p(h["kc"]), _p(h["vc"])
        s.m_prime, s.hNc_cap = h["m_prime"], h["kc"].shape[1]
        s.hkw, s.hvw, s.hraw_pos0 = _p(h["kw"]), _p(h["vw"]), _p(h["raw_pos0"])
        s.hR = h["kw"].shape[1] if h["kw"] is not None else 0
        s.hwindow, s.hsink = h["window"], _p(h["sink"])
        s.hsoftmax_scale = d ** -0.5 if h["scale"] is None else h["scale"]
        s.hout, s.hlse_out = _p(self.hout), _p(self.hlse)
        s.flags = L.STEP_FUSED_TAIL if fused_tail else 0
        self._desc = s
        self._lib = L.load()
        self._nws = self._lib.csa_hybrid_decode_step_workspace(s)
        # allocated zeroed: the step's control words must start at zero (every
        # call leaves them zero)
        self._ws = torch.zeros(max(self._nws, 1), dtype=torch.uint8, device=dev)
        self._wsp = self._ws.data_ptr()
        self._dev = dev
        self._inputs = (i, c, h, pos0)     # keep the tensors alive

    def run(self, stream=None):
        """Enqueue the step on `stream` (a raw hipStream_t; default: the
        current stream of the inputs' device)."""
        st = _stream(self._dev) if stream is None else stream
        L.check(self._lib.csa_hybrid_decode_step(self._desc, self._wsp, self._nws, st))
        return self

    def run_static(self, stream=None):
        """The same step through csa_hybrid_decode_step_static: its scratch is
        the library's static per-device array (no workspace of this object is
        used; calls that overlap on one device race)."""
        st = _stream(self._dev) if stream is None else stream
        L.check(self._lib.csa_hybrid_decode_step_static(self._desc, st))
        return self
