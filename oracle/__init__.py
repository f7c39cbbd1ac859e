"""Independent fp64 CPU oracle of the gated delta rule forward pass.

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or load anything here.
The product path (the HIP library and its Python binding) never does, and the
oracle shares no code, header, table or helper with it; both take their
inputs from the seeded generator module, which holds none of the method's
arithmetic.

* ``recurrence``  -- plain fp64 per-token recurrence in C (gdr_oracle.c),
                     OpenMP over the independent (batch, value-head) scans.
                     This is the definition the chunkwise method reproduces.
* ``chunk_form``  -- fp64 NumPy/SciPy chunkwise algorithm in the page's step
                     order, exposing gamma, A_kk, M, W, U, A_qk.
* ``ut_inverse_*``-- three forms of the UT inverse (triangular solve, Neumann
                     series, row iteration) that the pages state are equal.
* ``l2norm_rows`` -- fp64 row normaliser x * rsqrt(sum x^2 + 1e-6), the
                     reference for in-kernel q/k normalisation.

Pins (tests/test_oracle_*.py, CPU only): chunk form == recurrence for several
chunk sizes, closed forms (beta = 0 and g = 0; orthonormal keys; repeated
unit key; reset by g = -800; standard-basis keys with per-channel decay),
a Kronecker-product brute force on tiny shapes, segment splitting, joint
linearity, grouped-head equivalence, hand-derived golden values, and the
three UT inverse forms against each other, and the row normaliser against a
hand-derived row, its closed-form norm and the zero row.  No function here
is left unpinned.
"""
from .recurrence import build, num_threads, recurrence, recurrence_heads  # noqa: F401
from .chunk_form import (chunk_forward, decayed_dot, ut_inverse_neumann,  # noqa: F401
                         ut_inverse_rowloop, ut_inverse_solve)
from .l2norm import l2norm_rows  # noqa: F401
