"""fp64 CPU oracle for compensated block-sparse video attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or
runs this package: only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP path; both sides see the
same inputs through the `workloads` package, which holds no attention
arithmetic.

What it computes, each function citing the page passage it follows:

* `pooling`   - per-block means, key counts, first-order moments H_j, block
                spreads and e4m3 block copies (PISA, "Algorithme Central" and
                "Implementation Materielle": centroids, value sums and the
                per-block first-order matrices are precomputed).
* `routing`   - top-k on pooled scores, the LVSA window + rotating-anchor
                mask, and the Triage three-tier assignment.
* `attention` - dense softmax attention and the compensated rule
                o_t = N_t / D_t (PISA, "Algorithme Central") with exact,
                fp8-skim, centroid (zeroth-order) and per-block first-order
                Taylor terms inside one softmax normalisation.
* `e4m3`      - OCP fp8 e4m3 encode/decode from the format's definition.

Parity status: every function is pinned by CPU tests against closed forms,
invariants, library routines or brute force (see tests/test_oracle_*.py),
except the quality measure (relative L2 to dense), which is reported only:
parity unpinned.
"""

from . import e4m3, pooling, routing, attention  # noqa: F401
