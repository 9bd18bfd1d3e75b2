"""Oracle: a plain, slow, float64 CPU implementation of what the tree-packed
KDA path computes.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package.  The GPU library never routes through it,
and it shares no code with the HIP path (no kernels, helpers, tables or
pre/post-processing): the two meet only through the seeded inputs of
tree_packed_chunkwise_amd.synth.

Sources are the HARTS pages (arXiv 2608.28158): the devfeed.tech abstract,
the thelatestinai.com figure captions (Figures 1, 2, C.1, D.1-D.3) and the
zot.news summary.  The pages name KDA layers but print no recurrence; the
gated delta rule used here (per-channel decay, write strength beta, one
dk x dv state per head) is the reading fixed for this build and is stated in
oracle.kda.

Modules
  tree       rollout-tree conventions: offsets, trajectories, gather map
  kda        token-by-token recurrence, forward and reverse mode, over a
             path, a tree, and the trajectory-expanded tree
  chunkwise  the chunk form of the same recurrence, executed round by round
             over a packed plan (replay, handoff buffers), forward and reverse
  planner    the two-mode min-call planner, exhaustive search, and the
             canonical plan arrays
  gather     per-original-position log-prob recovery from compact logit rows
  attention  ancestor-masked softmax attention over the tree

Every function is pinned by tests under tests/ (test_oracle_*.py) against
closed forms, brute force, finite differences, exhaustive search or library
routines, as listed in each module.
"""
