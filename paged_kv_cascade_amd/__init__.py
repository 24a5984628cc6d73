"""MI355X-native paged-KV cascade decode attention.

Batched decode attention over a paged (block-table) KV cache on gfx950:
attention states (O, LSE) combined with the merge operator, split-KV with a
CPU load-balancing plan, and two-level / multi-level cascades.  The compute
path is the C-ABI library ``libpkc.so`` (hand-written HIP kernels, see
``include/pkc.h``); ``paged_kv_cascade_amd.api`` is a thin ctypes binding that
passes torch device pointers and torch's current stream through it.

Importing this package loads nothing; ``paged_kv_cascade_amd.api`` loads the
library and raises if it has not been built.
"""

__all__ = ["api", "workloads"]
