"""CPU oracle for block-sparse attention — test infrastructure, not product.

Plain, slow, obviously-correct numpy float64 statements of what the library
computes.  Only ``tests/``, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package; the HIP library
never calls it and shares no code with it.  Inputs are the arrays of the
seeded generator (float32 scores, bfloat16 bit patterns widened exactly to
float64); outputs are float64 (attention) or exact integers (masks, lists).

Modules:

* ``oracle.mask``      — top-k / threshold block masks and their compaction
  into per-row ascending lists (TileLang block-sparse Flash-Attention
  guide §3.1, §3.2, §4.4; XAttention guide, "algorithm flow", phase 3).
* ``oracle.attention`` — block-sparse prefill attention as a dense softmax
  over the token-level expansion of the block mask (same guide §5, §4.5),
  and sparse GQA decode over selected KV blocks (same guide §6–§6.2).
* ``oracle.heuristic`` — the split-count heuristic (same guide §6.3).
* ``oracle.xattn``     — the XAttention block-importance estimator: stride
  reshape (inverse mode), block sums of the reshaped softmax, and selection
  by cumulative weight with sink and diagonal (XAttention guide, "algorithm
  flow" phases 1-3).

Every function is pinned by tests against library routines, brute force,
closed forms and invariants (``tests/test_oracle_*.py``).
"""
