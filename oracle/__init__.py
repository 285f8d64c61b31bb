"""CPU oracle of the Medusa draft-and-verify step -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct implementation in float64 NumPy (exact
rational arithmetic for tree scores), written from the Medusa pages:

* "Medusa: Simple LLM Inference Acceleration Framework with Multiple Decoding
  Heads" (summary page): sections "MEDUSA Heads", "Tree Attention" (steps 1-6),
  "Typical Acceptance Scheme", "Optimized Tree Construction" (steps 1-4).
* "Accelerating LLM Inference with Speculative Decoding: Notes on Medusa":
  sections 3 "Tree Attention" and 4 "Optimized Tree Construction".
* "MEDUSA 精读": section 3 (draft tree, tree attention, verification) and
  section 6 (implementation checklist: KV-cache compaction).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product.  The two share only the seeded input generator in
``workloads/``, which holds none of the step's arithmetic.

Every function here is pinned by ``-m "not gpu"`` tests against values the
pages print, closed forms, invariants, library routines for special cases, or
brute force on tiny inputs (see ``tests/test_oracle_*.py``).
"""
