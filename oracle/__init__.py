"""fp64 CPU oracle for fused tiled scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP library (``tiled_attention_04_amd``), and it never
imports that package.

Sources (web pages; cited by title and section):

* "Building Flash Attention from Scratch in Pure NumPy" (martinuke0.github.io,
  2026-09-04) -- Step 1 (reference oracle), Step 2 (online softmax update),
  Step 3 (forward tile loops), Step 4 (backward with D = rowsum(dO*O)).
* "Build a FlashAttention-2 Inference Kernel from Scratch in Pure Python"
  (martinuke0.github.io, 2026-09-13) -- Step 2 (scale, then -inf masking),
  Step 3 (causal and sliding-window masks).
* "Build a FlashAttention Kernel with Online Softmax and KV Cache in Pure
  Python" (martinuke0.github.io, 2026-11-01) -- Steps 4-5 (single-token
  decode over a cache, naive reference).
* "Build a FlashAttention-2 Inference Kernel from Scratch in Pure Python",
  Extending It -- the paged KV cache (``decode_paged_ref``).
* "FlashAttention Algorithm > Worked Example" (mbrenndoerfer.com) -- Setup and
  Steps 1-3 (n=8, d=4, block 4 trace).

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
the pages print, closed forms, invariants, an independent library routine and
finite differences.  No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    allowed_mask,
    attention_ref,
    attention_rows_ref,
    attention_probs_ref,
    attention_tiled_ref,
    decode_ref,
    decode_paged_ref,
    attention_bwd_ref,
)
