"""Plain fp64 CPU oracle for paged-KV cascade decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls
this package, and the library has no CPU fallback.  The only callers are
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The oracle shares no code with the HIP path: it imports only
numpy and the Python standard library.

Sources (the four pages this method is described on):

* "Attention States and Recursive Attention" (FlashInfer tutorial):
  definitions of the generalised score s(I) and value v(I), the binary and
  n-ary merge operator, its commutativity and associativity, and the two
  applications (shared-prefix batch decode, KV sequence parallelism).
* "Cascade Inference: Memory Bandwidth Efficient Shared Prefix Batch
  Decoding" (FlashInfer blog, 2024-02-02): the same attention-state algebra,
  the singleton case, and the three-step cascade algorithm.
* "Paged attention" (Hugging Face Transformers docs): the varlen
  ``cu_seq_lens`` indexing example and the decode ``block_table`` /
  ``cache_seqlens`` example.
* "FlashInfer: Efficient and Customizable Attention Engine for LLM Inference
  Serving" (paper summary): attention composition (section A2), block-sparse
  KV storage and composable formats (A3), the load-balancing scheduler
  (A3, dynamic-aware runtime), and workspace sizing / split-K write-through
  (appendix D).

Modules:

* ``indexing``  -- token -> (page, slot) gather and cu_seq_lens maps.
* ``attention`` -- fp64 attention state of a query over a token set, and the
  batch decode / cascade results as ONE softmax over the union of each
  request's token sets (no merge operator on this path).
* ``merge``     -- the merge operator, used only to check the GPU merge and
  for the algebraic pins.
* ``plan``      -- the CPU load-balancing plan, step by step.
* ``fp8``       -- OCP E4M3 decoding of FP8 KV pools and the decode over the
  dequantised pools (paper summary, appendix F).

Every function here has at least one pin in ``tests/test_oracle_*.py``
against something other than itself (closed forms, worked examples printed
on the pages, a textbook routine, brute force).
"""

from . import indexing, attention, merge, plan, fp8  # noqa: F401
