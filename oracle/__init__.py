"""Plain fp64 CPU oracle for DeFT-style tree attention.  TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

Contents
  attention.py  the definition of tree-constrained attention, written out
                (per query: gather its root-to-node path KV through the block
                table, scaled dot products, softmax, PV), plus the per-chunk
                partial (O, m, l) convention and the log-sum-exp merge
  plan.py       a reference planner: flatten the tree, cut equal chunks,
                group the queries that see each chunk, build the bitmasks
                and each query's merge list
  io_model.py   KV read accounting (ideal unique bytes, naive per-query
                bytes, and the toy read counter of the DeFT Guide's simulator)

Every function cites the passage of the DeFT pages it follows.  Pins for each
are in tests/test_oracle_pins.py and tests/test_ref_plan.py.
"""
