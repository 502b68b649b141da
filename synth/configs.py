"""Workload descriptions (sizes, ratios, dtypes) for the CSA/HCA hot path.

The pages (DeepSeek-V4 summaries: hyper.ai "Method", aiboss88 "Technical
Principles") name the mechanisms but fix none of m, m', k, window, head
counts or dims; every constant below is a stated choice of this workload set.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # workload id, part of every seed
    dtype: str               # "f32" | "bf16": storage/compute dtype of q, k, v and caches
    mode: str                # "prefill" (raw tokens given) | "decode" (compressed caches given)
    B: int
    H: int                   # query heads; one shared KV head (MQA)
    d: int                   # head dim
    ctx: int                 # context length L (tokens seen so far, incl. the queries)
    Tq: int                  # query tokens per sequence; queries sit at positions ctx-Tq .. ctx-1
    # CSA (absent for HCA-only workloads)
    m: int = 0
    topk: int = 0
    window: int = 0
    HI: int = 0
    dI: int = 0
    qk_dtype: str = ""       # "f32" | "bf16" | "fp8" | "fp4"
    # HCA (absent for CSA-only workloads)
    m_hca: int = 0
    hca_window: int = 0
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def has_csa(self) -> bool:
        return self.m > 0

    @property
    def has_hca(self) -> bool:
        return self.m_hca > 0

    @property
    def pos0(self) -> int:
        return self.ctx - self.Tq

    @property
    def Nc(self) -> int:
        return self.ctx // self.m if self.m else 0

    @property
    def Nc_hca(self) -> int:
        return self.ctx // self.m_hca if self.m_hca else 0

    @property
    def scale(self) -> float:
        return self.d ** -0.5

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Tiny prefill: fp32, B=1, 1024 tokens, 4 query heads on 1 KV head, d=64.
# CSA m=4, top-32, window 64; indexer 2 heads x 32 dims; HCA m'=32 dense.
TINY = Workload(name="tiny_f32", wid=1, dtype="f32", mode="prefill", B=1, H=4, d=64,
                ctx=1024, Tq=1024, m=4, topk=32, window=64, HI=2, dI=32, qk_dtype="f32",
                m_hca=32)

# CSA prefill: bf16, 32K tokens, 64 heads, d=128, m=4 (8192 entries), top-512,
# window 128, indexer 4 heads x 64 dims.
CSA_PREFILL_32K = Workload(name="csa_prefill_32k", wid=2, dtype="bf16", mode="prefill", B=1,
                           H=64, d=128, ctx=32768, Tq=32768, m=4, topk=512, window=128,
                           HI=4, dI=64, qk_dtype="bf16")

# CSA decode: bf16 caches, B=64, context 131072 (32768 entries at m=4),
# 1 query token per sequence, top-1024, window 128.
CSA_DECODE_128K = Workload(name="csa_decode_128k", wid=3, dtype="bf16", mode="decode", B=64,
                           H=64, d=128, ctx=131072, Tq=1, m=4, topk=1024, window=128,
                           HI=4, dI=64, qk_dtype="bf16")

# HCA at 1M context, m'=128 -> 8192 entries, dense over completed blocks, sink.
HCA_1M_DECODE = Workload(name="hca_1m_decode", wid=4, dtype="bf16", mode="decode", B=16,
                         H=64, d=128, ctx=1 << 20, Tq=1, m_hca=128)
HCA_1M_PREFILL = Workload(name="hca_1m_prefill4k", wid=4, dtype="bf16", mode="decode", B=1,
                          H=64, d=128, ctx=1 << 20, Tq=4096, m_hca=128,
                          extra={"variant": 1})

# Hybrid CSA+HCA layer pair at 1M context, decode batch 8.  CSA m=4
# (262144 entries), top-2048, window 128; indexer QK in FP8 e4m3 (per-row
# scale) or FP4 e2m1 (per-32 E8M0 block scales); attention bf16; HCA m'=128.
HYBRID_1M_FP8 = Workload(name="hybrid_1m_fp8", wid=5, dtype="bf16", mode="decode", B=8,
                         H=64, d=128, ctx=1 << 20, Tq=1, m=4, topk=2048, window=128,
                         HI=4, dI=64, qk_dtype="fp8", m_hca=128)
HYBRID_1M_FP4 = HYBRID_1M_FP8.with_(name="hybrid_1m_fp4", qk_dtype="fp4")

WORKLOADS = {w.name: w for w in (TINY, CSA_PREFILL_32K, CSA_DECODE_128K, HCA_1M_DECODE,
                                 HCA_1M_PREFILL, HYBRID_1M_FP8, HYBRID_1M_FP4)}


def get(name: str) -> Workload:
    return WORKLOADS[name]
