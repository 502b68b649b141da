"""Host-side checks of the C ABI that need no GPU: every declared symbol is
exported, and invalid arguments are rejected with the right status before any
device work (the pointers used here are never dereferenced)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from sparse_attention_17_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "csa_mi355x.h")
FAKE = 0x100000          # aligned, never dereferenced: validation fails first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_\w+|hca_\w+)\s*\(", src)))


def test_header_declares_the_four_ops():
    names = declared_functions()
    for n in ("csa_compress", "csa_indexer_topk", "csa_sparse_attend", "hca_attend"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert set(names) == set(L.EXPORTS)


def test_version(lib):
    assert lib.csa_abi_version() == 1


def _compress(lib, **kw):
    a = dict(k=FAKE, v=FAKE, ki=None, gate=FAKE, pos_bias=None, B=1, T=64, d=128, dI=64, m=4,
             Nc_cap=16, dt=L.BF16, kc=FAKE, vc=FAKE, kic=None, stream=None)
    a.update(kw)
    return lib.csa_compress(*a.values())


def test_compress_validation(lib):
    assert _compress(lib, d=96) == L.UNSUPPORTED
    assert b"head dim" in lib.csa_last_error()
    assert _compress(lib, m=0) == L.INVALID_ARGUMENT
    assert _compress(lib, Nc_cap=15) == L.INVALID_ARGUMENT
    assert _compress(lib, k=None) == L.INVALID_ARGUMENT
    assert _compress(lib, k=FAKE + 4) == L.INVALID_ARGUMENT          # misaligned
    assert _compress(lib, ki=FAKE) == L.INVALID_ARGUMENT             # ki without kic
    assert _compress(lib, ki=FAKE, kic=FAKE, dI=48) == L.UNSUPPORTED
    assert _compress(lib, dt=L.FP8_E4M3) == L.UNSUPPORTED
    # nothing to do: succeeds without touching the device
    assert _compress(lib, B=0) == L.OK
    assert _compress(lib, T=3) == L.OK
    assert lib.csa_last_error() == b""


def test_compress_window_validation(lib):
    a = dict(k=FAKE, v=FAKE, ki=None, gate=FAKE, pos_bias=None, B=1, T=64, d=128, dI=64, m=4,
             width=8, Nc_cap=16, dt=L.BF16, kc=FAKE, vc=FAKE, kic=None, stream=None)
    call = lambda **kw: lib.csa_compress_window(*{**a, **kw}.values())
    assert call(width=3) == L.INVALID_ARGUMENT          # below m
    assert call(width=9) == L.INVALID_ARGUMENT          # above 2m
    assert b"width" in lib.csa_last_error()
    assert call(B=0) == L.OK


def _indexer(lib, **kw):
    a = dict(qi=FAKE, qi_scale=None, w=FAKE, kic=FAKE, kic_scale=None, pos0=FAKE, max_pos=1023,
             B=1, Tq=1, Nc_cap=256, HI=4, dI=64, m=4, topk=32, qk=L.BF16, idx=FAKE, score=None,
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return lib.csa_indexer_topk(*a.values())


def test_indexer_validation(lib):
    assert _indexer(lib, topk=0) == L.INVALID_ARGUMENT
    assert _indexer(lib, topk=4097) == L.INVALID_ARGUMENT
    assert _indexer(lib, HI=3) == L.UNSUPPORTED
    assert _indexer(lib, dI=48) == L.UNSUPPORTED
    assert _indexer(lib, max_pos=1027) == L.INVALID_ARGUMENT          # sees 257 > Nc_cap entries
    assert _indexer(lib, qk=L.FP8_E4M3) == L.INVALID_ARGUMENT         # scales missing
    assert _indexer(lib, qk=7) == L.INVALID_ARGUMENT
    assert _indexer(lib, qi=None) == L.INVALID_ARGUMENT
    need = lib.csa_indexer_topk_workspace(1, 1, 256, 4, 64, 32, L.BF16)
    assert need > 0
    assert _indexer(lib, ws=FAKE, ws_bytes=need - 1) == L.WORKSPACE_TOO_SMALL
    assert _indexer(lib, Tq=0) == L.OK


def _sparse(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, idx=FAKE, topk=256, kw=FAKE, vw=FAKE, raw_pos0=FAKE, R=128,
             pos0=FAKE, max_pos=4095, window=128, sink=None, scale=C.c_float(0.1), B=2, Tq=1,
             H=64, d=128, Nc_cap=1024, dt=L.BF16, out=FAKE, lse=None, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.csa_sparse_attend(*a.values())


def test_sparse_attend_validation(lib):
    assert _sparse(lib, H=129) == L.UNSUPPORTED
    assert _sparse(lib, d=32) == L.UNSUPPORTED
    assert _sparse(lib, topk=0) == L.INVALID_ARGUMENT
    assert _sparse(lib, window=-1) == L.INVALID_ARGUMENT
    assert _sparse(lib, kw=None) == L.INVALID_ARGUMENT
    assert _sparse(lib, R=0) == L.INVALID_ARGUMENT
    assert _sparse(lib, dt=L.FP4_E2M1) == L.UNSUPPORTED
    assert _sparse(lib, max_pos=-5) == L.INVALID_ARGUMENT
    assert _sparse(lib, scale=C.c_float(0.0)) == L.INVALID_ARGUMENT      # the scale must be > 0
    assert _sparse(lib, scale=C.c_float(-0.1)) == L.INVALID_ARGUMENT
    need = lib.csa_sparse_attend_workspace(2, 1, 64, 128, 256, 128)
    assert need > 0                                          # one decode token: split-KV partials
    assert _sparse(lib, ws=FAKE, ws_bytes=need - 1) == L.WORKSPACE_TOO_SMALL
    assert lib.csa_sparse_attend_workspace(1, 4096, 64, 128, 512, 128) == 0   # prefill: no split


def _hca(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, m_prime=128, Nc_cap=8192, kw=None, vw=None, raw_pos0=None,
             R=0, window=0, pos0=FAKE, max_pos=(1 << 20) - 1, sink=None, scale=C.c_float(0.1),
             B=16, Tq=1, H=64, d=128, dt=L.BF16, out=FAKE, lse=None, ws=None, ws_bytes=0,
             stream=None)
    a.update(kw)
    return lib.hca_attend(*a.values())


def test_hca_validation(lib):
    assert _hca(lib, m_prime=0) == L.INVALID_ARGUMENT
    assert _hca(lib, window=16) == L.INVALID_ARGUMENT          # window without a raw buffer
    assert _hca(lib, H=0) == L.UNSUPPORTED
    assert _hca(lib, scale=C.c_float(float("inf"))) == L.INVALID_ARGUMENT
    need = lib.hca_attend_workspace(16, 1, 64, 128, 8192, 128, 0)
    assert need == 32 * 16 * 64 * 130 * 4                      # 32 splits of 256 entries
    assert _hca(lib, ws=FAKE, ws_bytes=need - 1) == L.WORKSPACE_TOO_SMALL
    assert _hca(lib, B=0) == L.OK


WS_C, WS_H = 0x10000000, 0x20000000    # separate fake workspaces


def _hybrid(lib, csa=None, hca=None):
    c = dict(q=FAKE, kc=FAKE, vc=FAKE, idx=FAKE, topk=256, kw=FAKE, vw=FAKE, raw_pos0=FAKE, R=128,
             pos0=FAKE, max_pos=4095, window=128, sink=None, scale=C.c_float(0.1), B=2, Tq=1,
             H=64, d=128, Nc_cap=1024, dt=L.BF16, out=FAKE, lse=None, ws=WS_C, ws_bytes=1 << 26)
    h = dict(q=FAKE, kc=FAKE, vc=FAKE, m_prime=128, Nc_cap=8192, kw=None, vw=None, raw_pos0=None,
             R=0, window=0, pos0=FAKE, max_pos=(1 << 20) - 1, sink=None, scale=C.c_float(0.1),
             B=16, Tq=1, H=64, d=128, dt=L.BF16, out=FAKE + 0x1000, lse=None, ws=WS_H,
             ws_bytes=1 << 26)
    c.update(csa or {})
    h.update(hca or {})
    return lib.csa_hybrid_attend(*c.values(), *h.values(), None)


def test_hybrid_attend_validation(lib):
    # each part is validated as by its own entry point; the error names the part
    assert _hybrid(lib, csa=dict(topk=0)) == L.INVALID_ARGUMENT
    assert lib.csa_last_error().startswith(b"CSA part: topk")
    assert _hybrid(lib, hca=dict(m_prime=0)) == L.INVALID_ARGUMENT
    assert lib.csa_last_error().startswith(b"HCA part: m_prime")
    assert _hybrid(lib, hca=dict(d=96)) == L.UNSUPPORTED
    assert _hybrid(lib, csa=dict(scale=C.c_float(0.0))) == L.INVALID_ARGUMENT
    cn = lib.csa_sparse_attend_workspace(2, 1, 64, 128, 256, 128)
    hn = lib.hca_attend_workspace(16, 1, 64, 128, 8192, 128, 0)
    assert _hybrid(lib, csa=dict(ws_bytes=cn - 1)) == L.WORKSPACE_TOO_SMALL
    assert lib.csa_last_error().startswith(b"CSA part")
    assert _hybrid(lib, hca=dict(ws_bytes=hn - 1)) == L.WORKSPACE_TOO_SMALL
    assert lib.csa_last_error().startswith(b"HCA part")
    # the two workspaces must not overlap, nor the two outputs coincide
    assert _hybrid(lib, hca=dict(ws=WS_C + cn - 16)) == L.INVALID_ARGUMENT
    assert b"overlap" in lib.csa_last_error()
    assert _hybrid(lib, hca=dict(ws=WS_C - hn + 16)) == L.INVALID_ARGUMENT
    assert _hybrid(lib, hca=dict(out=FAKE)) == L.INVALID_ARGUMENT
    assert b"same buffer" in lib.csa_last_error()
    # both parts empty: nothing to do
    assert _hybrid(lib, csa=dict(B=0), hca=dict(Tq=0)) == L.OK


def _proj(lib, **kw):
    a = dict(o=FAKE, w=FAKE, T=64, H=64, d=128, G=8, dg=1024, dt=L.BF16, y=FAKE, stream=None)
    a.update(kw)
    return lib.csa_grouped_out_proj(*a.values())


def test_grouped_out_proj_validation(lib):
    assert _proj(lib, G=3) == L.INVALID_ARGUMENT                # G must divide H
    assert _proj(lib, H=4, d=8, G=1) == L.UNSUPPORTED           # K = 32 not a multiple of 64
    assert _proj(lib, dg=100) == L.UNSUPPORTED
    assert _proj(lib, dt=L.FP8_E4M3) == L.UNSUPPORTED
    assert _proj(lib, y=None) == L.INVALID_ARGUMENT
    assert _proj(lib, o=FAKE + 8) == L.INVALID_ARGUMENT         # misaligned
    assert _proj(lib, T=1 << 20) == L.INVALID_ARGUMENT          # o over 2 GiB
    assert _proj(lib, T=0) == L.OK


def test_kv8_validation(lib):
    a = dict(q=FAKE, k8=FAKE, krope=FAKE, kscale=FAKE, v8=FAKE, vscale=FAKE, m_prime=128,
             Nc_cap=8192, kw=None, vw=None, raw_pos0=None, R=0, window=0, pos0=FAKE,
             max_pos=(1 << 20) - 1, sink=None, scale=C.c_float(0.1), B=16, Tq=1, H=64, d=128,
             out=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 26, stream=None)
    call = lambda **kw: lib.hca_attend_kv8(*{**a, **kw}.values())
    assert call(d=64) == L.UNSUPPORTED                       # built for d = 128
    assert call(vscale=None) == L.INVALID_ARGUMENT           # v8 without its scales
    assert call(krope=None) == L.INVALID_ARGUMENT
    assert call(B=0) == L.OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        L.load()


def test_decode_step_struct_layout(tmp_path):
    # the ctypes mirror must match csa_decode_step_t field for field: compile a
    # C program against the header that prints every field's offset
    from sparse_attention_17_amd._lib import DecodeStepDesc
    names = [f[0] for f in DecodeStepDesc._fields_]
    prog = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "csa_mi355x.h"', 'int main(void) {',
             '  printf("size %zu\\n", sizeof(csa_decode_step_t));']
    lines += [f'  printf("{n} %zu\\n", offsetof(csa_decode_step_t, {n}));' for n in names]
    lines += ['  return 0;', '}']
    prog.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)],
                   check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True,
                                                   check=True).stdout.splitlines())
    assert int(got["size"]) == C.sizeof(DecodeStepDesc)
    for n in names:
        assert int(got[n]) == getattr(DecodeStepDesc, n).offset, n


def test_decode_step_validation(lib):
    from sparse_attention_17_amd._lib import DecodeStepDesc
    s = DecodeStepDesc()
    s.B, s.pos0, s.max_pos, s.H, s.d, s.dt = 2, FAKE, 1023, 8, 128, L.BF16
    s.qi, s.w, s.kic, s.HI, s.dI, s.m, s.topk, s.qk_dt, s.idx_out = FAKE, FAKE, FAKE, 4, 64, 4, 32, L.BF16, FAKE
    s.q, s.kc, s.vc, s.Nc_cap, s.window, s.softmax_scale, s.out = FAKE, FAKE, FAKE, 256, 0, 0.1, FAKE
    s.hq, s.hkc, s.hvc, s.m_prime, s.hNc_cap, s.hsoftmax_scale, s.hout = FAKE, FAKE, FAKE, 128, 8, 0.1, FAKE + 256
    need = lib.csa_hybrid_decode_step_workspace(C.byref(s))
    assert need > 0
    assert lib.csa_hybrid_decode_step(C.byref(s), FAKE, need - 1, None) == L.WORKSPACE_TOO_SMALL
    s.HI = 3
    assert lib.csa_hybrid_decode_step(C.byref(s), FAKE, need, None) == L.UNSUPPORTED
    assert b"indexer part" in lib.csa_last_error()
    s.HI, s.softmax_scale = 4, -1.0
    assert lib.csa_hybrid_decode_step(C.byref(s), FAKE, need, None) == L.INVALID_ARGUMENT
    assert b"CSA part" in lib.csa_last_error()
    s.softmax_scale, s.hkc = 0.1, None
    assert lib.csa_hybrid_decode_step(C.byref(s), FAKE, need, None) == L.INVALID_ARGUMENT
    assert b"HCA part" in lib.csa_last_error()
    s.hkc, s.hout = FAKE, s.out
    assert lib.csa_hybrid_decode_step(C.byref(s), FAKE, need, None) == L.INVALID_ARGUMENT
    assert b"same buffer" in lib.csa_last_error()
    assert lib.csa_hybrid_decode_step(None, FAKE, need, None) == L.INVALID_ARGUMENT


def test_decode_step_flags_undefined_bits(lib):
    from sparse_attention_17_amd._lib import DecodeStepDesc
    s = DecodeStepDesc()
    s.B, s.H, s.Nc_cap, s.m_prime, s.topk, s.flags = 1, 8, 64, 8, 4, 2
    assert lib.csa_hybrid_decode_step(C.byref(s), None, 0, None) == L.INVALID_ARGUMENT
    assert b"flags" in lib.csa_last_error()


def test_static_step_validation(lib):
    # rejected before any device work: no step, or a step whose scratch needs
    # more than the static array holds
    from sparse_attention_17_amd._lib import DecodeStepDesc
    assert lib.csa_hybrid_decode_step_static(None, None) == L.INVALID_ARGUMENT
    s = DecodeStepDesc()
    s.B, s.pos0, s.max_pos, s.H, s.d, s.dt = 64, FAKE, (1 << 23) * 4 - 1, 64, 128, L.BF16
    s.HI, s.dI, s.m, s.topk, s.qk_dt, s.Nc_cap = 4, 64, 4, 2048, L.FP8_E4M3, 1 << 23
    s.m_prime, s.hNc_cap, s.window = 128, 1 << 18, 128
    assert lib.csa_hybrid_decode_step_workspace(C.byref(s)) > 64 << 20
    assert lib.csa_hybrid_decode_step_static(C.byref(s), None) == L.WORKSPACE_TOO_SMALL
    assert b"static array" in lib.csa_last_error()
