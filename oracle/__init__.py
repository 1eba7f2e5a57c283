"""fp64 CPU oracle for the CompKV decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product library
(``block_sparse_kv_stats_amd``) never imports it, and it imports nothing from
the product library: the two share no code, tables or helpers.

Source of every formula: the CompKV page (onedev.kr/papers/157), sections
"How it works" (어떻게 동작하나), "What differs" (무엇과 다른가) and
"How to use it" (어떻게 쓰나). Where that page leaves a step open, the reading
taken is stated at the function that takes it.

Modules:
  compkv -- the method: block summaries, block scores, selection, compensated
            attention, dense attention, the streaming (per-step) oracle.
  theory -- the exact quantities of the page's analysis (block masses,
            logit variances, the KL selection loss and its second-order
            surrogate, brute-force subset search) used only to pin compkv.

Parity status: every function in ``compkv`` is pinned by a CPU test in
``tests/test_oracle_pins.py`` except the grouping of coordinates into
contiguous groups for 1 < r < d, which the page does not fix (partly
pinned: within-group permutation invariance and the r = 1 / r = d closed
forms).
"""
