"""CPU oracle for tree-structured decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import or run anything in this package. The product path (the HIP library
and its Python binding) never calls it, and it shares no code with them.

* ``tree_attention``: the plain fp64 definition of what the decode step
  computes (DeFT reading notes, "tree attention definition"; FastTree review,
  section 3, the self-attention formula).
* ``planner_ref``: a plain-Python re-derivation of the host planner (FastTree
  review, section 3.2, Algorithm 1 and its cost model; section 3.3, long-context
  splitting) that produces the same tables the C-ABI library exports.
"""
