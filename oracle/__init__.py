"""CPU oracle for one EAGLE-3 speculative-decoding step.  TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the step computes, written
from the pages' statement of the method (cited per function by page title and
section).  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU
baseline leg may import it.  It shares no code with the HIP path and never
imports it; the product path must never route through it.

Modules
  numerics  storage rounding, softmax / log-sum-exp, the fp32 decision helpers
            and the integer inverse-CDF sampler
  llama     the LLaMA-shaped target forward (tree-masked or causal) and the
            EAGLE-3 draft head
  tree      tree mask, depths, the static-branching builder and the dynamic
            (confidence-ranked) builder
  accept    greedy longest-path acceptance, chain rejection sampling and
            level-by-level rejection sampling over a tree
  step      KV compaction and the vanilla / speculative driver loops
  paged     block-table slot mapping, per-request draft lengths and the verify
            batch's index bookkeeping
  ttt       training-time-test attention (causal native keys + diagonal simulated keys)

Every function is pinned by a test in tests/test_oracle_*.py.  One of them
computes a reading rather than a formula the pages print:
  tree.build_dynamic_tree  (the frontier / re-rank policy of a step the pages
                            name but do not spell out; pinned against that
                            reading by an independent enumeration of the
                            candidates, by its k = 1 and depth-1 reductions
                            to the greedy chain and the top-k, and by a
                            hand-worked case; no page gives another engine's
                            policy to compare it with)
"""
