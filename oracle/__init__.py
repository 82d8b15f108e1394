"""fp64 CPU oracle for decode attention over a prefix-shared KV tree.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the test suite, the smoke check of the
package entry point and the CPU-baseline leg of the benchmark use it.  It
shares no code with the HIP path and never reads the tree under test or the
device chunk pool; its only inputs are the seeded workload arrays.

Modules
  attention  the attention result per sequence, written as its plain
             definition (softmax of scaled dot products, fp64), plus the
             partial / merge equations of the ChunkAttention page (Knowl 3) and
             the result assembled from them over any cover of a context by
             disjoint pieces, used to pin the algebra the kernels rely on.
  sharing    which chunks a prefix tree stores once: the plain definition
             for insertion-built trees, and a small reference model of the
             arrival / decode-append / departure rules (Knowl 1) for dynamic
             operation sequences; plus the closed forms of Knowl 4.

Every function is pinned by tests that do not re-type its formula (brute
force, closed forms, special cases, invariances); see the test modules named
test_oracle_*.
"""
