"""CPU oracle for fine-grained-scaled FP8 GEMM (NumPy, float64).

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import, call or execute anything in this
package.  The HIP library never calls it and has no CPU fallback; the two
share no code.  Each function cites the passage of the pages it follows.

Pins: every function here is checked by `-m "not gpu"` tests against facts the
pages and the mathematics fix (closed forms, hand-derived values under
tests/golden/, exact rational brute force, exact special cases).  No function
is left "parity unpinned".
"""
from . import activation, backward, e4m3, gemm, routing, scaling  # noqa: F401
