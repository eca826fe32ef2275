"""fp64 CPU oracle for split-KV decode attention and its work plan.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package.  The product path
(the C-ABI library and its Python binding) never calls into it, and it shares
no code with that path: no kernels, tables, helpers or pre/post-processing.

Modules
-------
attention  the plain softmax-attention definition over a paged KV cache, the
           per-piece partial state and the log-sum-exp merge identity.
planner    the Stream-K work split (equal tile chunks, one per compute unit)
           serialised to the same byte layout the C library emits, plus a
           list-scheduling makespan model for the tail-effect example.
"""
