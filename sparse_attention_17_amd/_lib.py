"""ctypes loader for libcsa_mi355x.so (built in-tree by ``build.py``).

Loading fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa_mi355x.so")

# status codes (csa_status_t)
OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, DEVICE_ERROR = range(5)
# csa_dtype_t
F32, BF16, FP8_E4M3, FP4_E2M1 = range(4)
# csa_decode_step_t.flags
STEP_FUSED_TAIL = 1

_P = C.c_void_p
_I = C.c_int
_SZ = C.c_size_t


class DecodeStepDesc(C.Structure):
    """Mirror of csa_decode_step_t (include/csa_mi355x.h), field for field."""
    _fields_ = [
        ("B", _I), ("pos0", _P), ("max_pos", _I), ("H", _I), ("d", _I), ("dt", _I),
        ("qi", _P), ("qi_scale", _P), ("w", _P), ("kic", _P), ("kic_scale", _P),
        ("HI", _I), ("dI", _I), ("m", _I), ("topk", _I), ("qk_dt", _I), ("idx_out", _P),
        ("q", _P), ("kc", _P), ("vc", _P), ("Nc_cap", _I), ("kw", _P), ("vw", _P),
        ("raw_pos0", _P), ("R", _I), ("window", _I), ("sink", _P), ("softmax_scale", C.c_float),
        ("out", _P), ("lse_out", _P),
        ("hq", _P), ("hkc", _P), ("hvc", _P), ("m_prime", _I), ("hNc_cap", _I), ("hkw", _P),
        ("hvw", _P), ("hraw_pos0", _P), ("hR", _I), ("hwindow", _I), ("hsink", _P),
        ("hsoftmax_scale", C.c_float), ("hout", _P), ("hlse_out", _P),
        ("flags", C.c_uint),
    ]


EXPORTS = {
    "csa_abi_version": (_I, []),
    "csa_last_error": (C.c_char_p, []),
    "csa_compress": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "csa_compress_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P,
                                 _P]),
    "csa_indexer_topk_workspace": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "csa_indexer_topk": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I,
                              _P, _P, _P, _SZ, _P]),
    "csa_sparse_attend_workspace": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "csa_sparse_attend": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _P, _I, _I, _P, C.c_float,
                               _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_workspace": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "hca_attend": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P, C.c_float,
                        _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa_sparse_attend_kv8": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _I, _P, _I, _I, _P,
                                   C.c_float, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_kv8": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P,
                            C.c_float, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa_hybrid_attend": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _I, _P, _I, _I, _P, C.c_float,
                               _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ,
                               _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P, C.c_float,
                               _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "csa_hybrid_decode_step_workspace": (_SZ, [C.POINTER(DecodeStepDesc)]),
    "csa_hybrid_decode_step": (_I, [C.POINTER(DecodeStepDesc), _P, _SZ, _P]),
    "csa_hybrid_decode_step_static": (_I, [C.POINTER(DecodeStepDesc), _P]),
    "csa_grouped_out_proj": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "csa_profile_enable": (None, [_I]),
    "csa_profile_reset": (None, []),
    "csa_profile_query": (_I, [C.c_char_p, C.POINTER(C.c_int), C.POINTER(C.c_double)]),
    "csa_profile_counter": (_I, [C.c_char_p, C.POINTER(C.c_ulonglong), _I]),
}



_lib = None


class CsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_17_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status: int) -> None:
    if status != OK:
        raise CsaError(status, load().csa_last_error().decode())
