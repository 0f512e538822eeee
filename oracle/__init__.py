"""CPU oracle for the CSA / HCA hybrid compressed attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only the test-suite, the package smoke check and
the ``cpu_baseline`` leg of the benchmark use it.  It shares no code with the
HIP library or its Python binding; the only thing the two sides have in common
is the seeded input generator module (random numbers and shapes, no method
arithmetic).

The oracle is plain, slow and written to be checked by eye against the pages:
float64 NumPy arithmetic everywhere except at the rounding points the method
defines (fp32 intermediate, bf16, FP8 e4m3fn, FP4 e2m1 with e8m0 block scales),
which are emulated bit-exactly.

Sources (cited below by the tag in brackets):

* [Notes] "DeepSeek V4: Towards Highly Efficient Million Token Context
  Intelligence" -- reading notes on the technical report (papers.chlience.com).
  §7 "CSA" (compressor, lightning indexer, top-k, shared-KV MQA, sliding
  window), §8 "HCA" (non-overlap compressor equations, compress_ratio table),
  §9 "CSA/HCA other details" (sink, KV precision, FP4 indexer, BF16 scores).
* [HF] "DeepSeek-V4: a million-token context that agents can actually use"
  (Hugging Face blog), section "Hybrid attention: CSA and HCA".
* [OCP-FP8] OCP 8-bit Floating Point Specification (OFP8), E4M3 encoding.
* [OCP-MX] OCP Microscaling Formats (MX) Specification v1.0, MXFP4.

Modules:
  codecs    -- bf16 / e4m3fn / e2m1 / MXFP4 / FP8-entry encode and decode
  compress  -- softmax-gated pooling (overlap CSA, non-overlap HCA)
  indexer   -- lightning-indexer scores and top-k selection
  attend    -- CSA and HCA core attention with the sliding-window branch
  pipeline  -- the decode / prefill steps chained from the four operations

Parity status per function is stated in each module header.  The readings
adopted where the pages are silent are listed in the repository design notes.
"""

from . import codecs, compress, indexer, attend, pipeline  # noqa: F401
from .codecs import KV, Idx  # noqa: F401
