"""CPU oracle for pre-RoPE KV injection with Chunked RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code with the HIP library (``pre_rope_kv_amd``) and imports nothing from it;
it depends on NumPy alone.

What it computes (page: "InferScale: GPU-Native KV Injection for Personalized
LLM Serving", Pith review of arXiv 2607.27090):

* "What carries the argument" and "The pith": each retrieved fact's keys are
  stored before rotary position encoding and rotated to their serving-time
  positions when they are injected; values are injected unchanged.
* "Referee Report", Summary: the rotated K and the V are scatter-copied into a
  vLLM paged KV cache (PagedAttention, reference [6]) through the block table.
* "Axiom & Free-Parameter Ledger", axiom on RoPE (R_a^T R_b = R_{b-a},
  Theorem 6 / section 5.1): rotation by position is a relocation.
* "Core claim" / Theorem 3: injecting KV at the intended positions equals
  prompt-injecting the same tokens (checked with brute-force attention).
* "Referee Report", Summary and Figure 2: facts are retrieved by their
  embeddings before injection (exact top-k by inner product, `retrieve`).

Precision: every floating-point step is float64; the single rounding to
bfloat16 is round-to-nearest-even.  The pages fix neither the rotation
convention nor the cache layout; the readings taken are stated in the module
docstrings.

Pinning: each function is pinned by tests that do not reuse its code
(closed forms, hand-worked golden fixtures, brute force, library routines and
invariants).  No function here is "parity unpinned".
"""

from . import attention, bf16, inject, paged, retrieve, rope  # noqa: F401
