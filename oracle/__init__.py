"""CPU oracle for token-tree attention and token-tree verification.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, float64 statement
of what the GPU path computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path (the HIP library
and its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product.

Sources (web pages; section names as printed on them):
  [guide]   "SpecInfer Guide: Tree-Based Speculative LLM Serving" (aifetchly blog)
  [chapter] "Inference Optimization Techniques: Speed and Efficiency" (aicomputerinstitute)
  [cohere]  Cohere's blog post on hardware-aware dynamic speculative decoding

Readings taken where the pages are silent or garbled are listed in the
design notes; each function names the one it relies on.

Modules:
  tree       ancestor walk, topology mask, tree validation
  attention  masked tree attention over a paged prefix KV cache
  verify     greedy and stochastic tree verification, linear speculative decoding
  kv         accepted-path KV compaction
  construct  token-tree construction: merge of candidates, top-k expansion
  pool       paged speculative-block allocation and release
  budget     expected acceptance length of a tree, goodput and the tree-size table

Pins: every function here is checked by tests marked "not gpu" against values
the pages print, closed forms, library routines on special cases and brute
force on tiny inputs (tests/test_oracle_*.py).
"""
# Per-request status flags (bitwise OR).  They mirror the error contract of the
# C interface so that malformed inputs can be compared request by request.
BAD_PARENT = 1      # parent[0] != -1, or parent[i] outside [0, i)
BAD_NNODES = 2      # n_nodes outside [1, n_max]
BAD_KV = 4          # prefix/positions outside the block table, or a block id outside the pool
NONFINITE = 8       # a logit row that is read holds NaN or +-inf
BAD_TOKEN = 16      # a child token outside [0, vocab) (stochastic verification)
BAD_PATH = 32       # accepted-path description that is not a root path of increasing node ids
TREE_OVERFLOW = 128 # a constructed tree would exceed n_max nodes
BAD_LEN = 256       # a candidate length, frontier count or frontier node id out of range
POOL_EXHAUSTED = 512  # the block pool cannot serve an allocation, or a release would overfill it
BAD_PROB = 1024     # an acceptance probability that is NaN or outside [0, 1] (tree-budget calibration)

from . import tree, attention, verify, kv, construct, pool, budget  # noqa: E402,F401
