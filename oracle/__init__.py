"""CPU oracle for block-sparse attention and its mean-pool top-k mask builder.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import or run anything here.
The GPU library never calls this code and shares none of its arithmetic.

Everything is plain numpy in float64 on the bf16-rounded inputs (upcast
exactly).  Page abbreviations (BSA-DiT, MC-Sparse summary) are defined in the
`workloads` package docstring.

* `attention`  - the masked-softmax definition of block-sparse attention.
* `builder`    - mean-pool / block-score / prior-union / top-k selection, and
                 the density -> per-row count plan.

Pins (tests/test_oracle_*.py) tie both to facts other than this code: torch's
float64 scaled_dot_product_attention on all-ones masks, closed forms (Q = 0,
V constant, a hand-worked two-token case), invariants, and brute-force subset
enumeration for the selector.  No function here is "parity unpinned".
"""
from . import attention, builder  # noqa: F401
