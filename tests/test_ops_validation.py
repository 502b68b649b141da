"""The torch wrappers reject wrong dtypes and shapes before anything reaches
the C ABI (which sees only pointers and cannot check them).  CPU tensors are
enough: the checks run before the device check."""
import pytest
import torch

from sparse_attention_17_amd import ops


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_compress_rejects():
    k = t(2, 64, 128)
    with pytest.raises(ValueError, match="v must"):
        ops.compress(k, t(2, 64, 64), None, f32(128), 4)
    with pytest.raises(ValueError, match="gate must be float32"):
        ops.compress(k, k, None, t(128), 4)
    with pytest.raises(ValueError, match="ki must"):
        ops.compress(k, k, t(2, 32, 64), f32(128), 4)
    with pytest.raises(ValueError, match="pos_bias"):
        ops.compress(k, k, None, f32(128), 4, pos_bias=f32(5))


def test_indexer_rejects():
    B, Tq, HI, dI, N = 2, 3, 4, 64, 100
    ok = dict(qi=t(B, Tq, HI, dI), w=f32(B, Tq, HI), kic=t(B, N, dI), pos0=i32(B), m=4, topk=8,
              max_pos=10)
    with pytest.raises(ValueError, match="pos0 must be int32"):
        ops.indexer_topk(**{**ok, "pos0": torch.zeros(B, dtype=torch.int64)})
    with pytest.raises(ValueError, match="pos0 must have shape"):
        ops.indexer_topk(**{**ok, "pos0": i32(B + 1)})
    with pytest.raises(ValueError, match="w must be float32"):
        ops.indexer_topk(**{**ok, "w": t(B, Tq, HI)})
    with pytest.raises(ValueError, match="kic must"):
        ops.indexer_topk(**{**ok, "kic": t(B, N, 32)})
    with pytest.raises(ValueError, match="kic must be torch.float32"):    # qi's dtype sets the format
        ops.indexer_topk(**{**ok, "qi": f32(B, Tq, HI, dI)})
    with pytest.raises(ValueError, match="FP8 needs"):
        ops.indexer_topk(**{**ok, "qi": t(B, Tq, HI, dI, dtype=torch.uint8),
                            "kic": t(B, N, dI, dtype=torch.uint8)}, qk_dtype="fp8")
    with pytest.raises(ValueError, match="kic_scale must have shape"):
        ops.indexer_topk(**{**ok, "qi": t(B, Tq, HI, dI, dtype=torch.uint8),
                            "kic": t(B, N, dI, dtype=torch.uint8)}, qk_dtype="fp8",
                         qi_scale=f32(B, Tq, HI), kic_scale=f32(B, N + 1))
    with pytest.raises(ValueError, match="qi_scale must"):
        ops.indexer_topk(**{**ok, "qi": t(B, Tq, HI, dI // 2, dtype=torch.uint8),
                            "kic": t(B, N, dI // 2, dtype=torch.uint8)}, qk_dtype="fp4",
                         qi_scale=t(B, Tq, HI, 1, dtype=torch.uint8),
                         kic_scale=t(B, N, 2, dtype=torch.uint8))


def test_attend_rejects():
    B, Tq, H, d, N = 2, 1, 8, 128, 50
    ok = dict(q=t(B, Tq, H, d), kc=t(B, N, d), vc=t(B, N, d), idx=i32(B, Tq, 16), pos0=i32(B),
              max_pos=199, window=0)
    with pytest.raises(ValueError, match="idx must be int32"):
        ops.sparse_attend(**{**ok, "idx": torch.zeros(B, Tq, 16, dtype=torch.int64)})
    with pytest.raises(ValueError, match="idx must have shape"):
        ops.sparse_attend(**{**ok, "idx": i32(B, Tq + 1, 16)})
    with pytest.raises(ValueError, match="kc must"):
        ops.sparse_attend(**{**ok, "kc": t(B, N, 64)})
    with pytest.raises(ValueError, match="vc must"):
        ops.sparse_attend(**{**ok, "vc": f32(B, N, d)})
    with pytest.raises(ValueError, match="sink must"):
        ops.sparse_attend(**ok, sink=f32(H + 1))
    with pytest.raises(ValueError, match="window > 0 needs"):
        ops.sparse_attend(**{**ok, "window": 4})
    with pytest.raises(ValueError, match="pos0 must be int32"):
        ops.hca_attend(ok["q"], ok["kc"], ok["vc"], 4, torch.zeros(B, dtype=torch.int64), 199)
    with pytest.raises(ValueError, match="kw must"):
        ops.hca_attend(ok["q"], ok["kc"], ok["vc"], 4, ok["pos0"], 199, window=2,
                       kw=t(B, 8, 64), vw=t(B, 8, 64), raw_pos0=i32(B))


def test_kv8_and_pair_reject():
    B, Tq, H, d, N = 2, 1, 8, 128, 50
    q = t(B, Tq, H, d)
    u8 = lambda *s: t(*s, dtype=torch.uint8)  # noqa: E731
    cache = (u8(B, N, d // 2), t(B, N, d // 2), f32(B, N), u8(B, N, d), f32(B, N))
    with pytest.raises(ValueError, match="krope must"):
        ops.hca_attend_kv8(q, (cache[0], f32(B, N, d // 2)) + cache[2:], 128, i32(B), 199)
    with pytest.raises(ValueError, match="v8 and vscale"):
        ops.hca_attend_kv8(q, cache[:3] + (cache[3], None), 128, i32(B), 199)
    with pytest.raises(ValueError, match="vscale must"):
        ops.sparse_attend_kv8(q, cache[:4] + (f32(B, N + 1),), i32(B, Tq, 16), i32(B), 199, 0)
    csa = dict(q=q, kc=t(B, N, d), vc=t(B, N, d), idx=i32(B, Tq, 16), pos0=i32(B), max_pos=199,
               window=0)
    hca = dict(q=q, kc=t(B, N, d), vc=t(B, N, d), m_prime=128, pos0=i32(B), max_pos=199)
    with pytest.raises(ValueError, match="idx must be int32"):
        ops.hybrid_attend({**csa, "idx": f32(B, Tq, 16)}, hca)
    with pytest.raises(ValueError, match="sink must"):
        ops.hybrid_attend(csa, {**hca, "sink": f32(3)})


def test_projection_rejects():
    with pytest.raises(ValueError, match="same dtype"):
        ops.grouped_out_proj(t(4, 8, 128), f32(2, 128, 512))
    with pytest.raises(ValueError, match="w must be"):
        ops.grouped_out_proj(t(4, 8, 128), t(2, 128, 256))
