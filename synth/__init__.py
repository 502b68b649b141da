"""Seeded synthetic inputs for the CSA/HCA hot path.

This package is shared by the oracle-side tests and the GPU-side tests/bench.
It holds only workload descriptions, seeded random draws, dtype rounding and
the FP8/FP4 *encoders* that turn drawn values into the codes the indexer
consumes.  It holds none of the attention method's arithmetic (no pooling,
scoring, selection or softmax over keys); those live separately in the oracle
and in the HIP kernels.
"""
from .configs import WORKLOADS, Workload, get  # noqa: F401
from .inputs import make_inputs, rng_for  # noqa: F401
