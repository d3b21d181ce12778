"""CPU oracle for SegPagedAttention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The library (sparse_attention_segmentpagetable_amd) never does;
the two share no code. Inputs come from the seeded generators in `workloads`.

attention.py  O1: attention as its plain definition -- dense fp64 scores, an
              explicit per-head visibility mask, softmax (plus a scalar-loop
              variant and a blocked online-softmax variant for cross-checks).
layout.py     O2: the SegmentPageTable ints and the expected page-pool bytes,
              written out from the retention and packing rules.

Every function is pinned by tests/test_oracle_*.py against closed forms, a
library routine, brute force or values the pages print; none is "parity
unpinned".
"""
