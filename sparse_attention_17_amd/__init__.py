"""CSA / HCA hybrid-attention hot path for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI declared in
include/csa_mi355x.h (libcsa_mi355x.so, built in-tree by ``build.py``);
``ops`` marshals torch tensors into those calls.
"""
from . import ops  # noqa: F401
from ._lib import CsaError, load  # noqa: F401
