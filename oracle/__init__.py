"""Plain, slow, fp64 CPU oracle for the CSA/HCA hybrid attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path (the HIP library, its
C ABI and the Python binding in ``sparse_attention_17_amd``) imports, links or
calls anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP path; the two meet only in the seeded inputs of
``synth``.

Sources (DeepSeek-V4 summary pages):
  * hyper.ai summary, section "Method", CSA paragraph: every m tokens are
    compressed into one entry with learnable compression weights and
    positional biases; a lightning indexer picks the top-k entries; core
    attention is MQA with shared keys and values.
  * same page, HCA paragraph: compression at m' >> m, non-overlapping, dense
    attention over the compressed entries; both mechanisms carry a sliding
    window branch.
  * same page, CSA paragraph: a grouped output projection follows the core
    attention (``proj``).
  * same page, efficiency paragraph, and aiboss88 "Technical Principles"
    (CSA and FP4 bullets): FP4 indexer QK path, FP8 for extra dynamic range,
    sliding window plus attention sink in CSA.
The pages give no equations; the concrete forms (softmax-gated pooling, the
ReLU-weighted indexer score, one softmax over selected entries + window +
sink) are the readings recorded in the design notes, and each function below
states the one it implements.

Parity pins (tests marked ``not gpu``) tie every function to something other
than itself: format definitions and torch's own float8 decoder, closed forms
of the pooling, brute-force sorts, and PyTorch's scaled_dot_product_attention
in float64 for the dense special cases.
"""
from . import formats, csa, hca, proj  # noqa: F401
