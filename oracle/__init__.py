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

Pins (tests/test_oracle_pins.py, CPU only), one or more per function:

* ``recurrence``       -- hand-derived golden values (tests/golden/), closed
                          forms (beta = 0 and g = 0; orthonormal keys;
                          repeated unit key; reset by g = -800;
                          standard-basis keys with per-channel decay), a
                          Kronecker-product brute force on tiny shapes,
                          segment splitting, joint linearity, grouped-head
                          equivalence with explicit repeat_interleave, and
                          (linear rule) the page's masked quadratic form.
* ``recurrence_heads`` -- every (b, hv) scan, and a cut T, equal the
                          recurrence run on all heads at once bit for bit;
                          the modulo grouping must differ.
* ``chunk_forward``    -- equals the recurrence for chunk sizes 1, 16, 64,
                          128 and T, with scalar and per-channel decay,
                          grouped heads, an initial state and ragged T.
* ``decayed_dot``      -- a triple loop over its definition, and the
                          factored (x k^T) * exp(gamma_i - gamma_j) form.
* ``ut_inverse_*``     -- the triangular solve, the Neumann series and the
                          row iteration agree (three forms the pages give).
* ``l2norm_rows``      -- a hand-derived row, the closed-form norm of any
                          output row, the kept direction and the zero row.

Property tests (tests/test_properties.py, Hypothesis on tiny shapes) add,
for ``recurrence``, ``chunk_forward`` and the ``ut_inverse_*`` forms: the
chunk form at any chunk length, the Kronecker form of both rules, key and
value channel relabelling, a cut anywhere with the state carried, batch
independence, linearity in the scale, the closed form at beta = 0, the
linear rule's quadratic form, and the inverses' agreement on any size.
"""
from .recurrence import build, num_threads, recurrence, recurrence_heads  # noqa: F401
from .chunk_form import (chunk_forward, decayed_dot, ut_inverse_neumann,  # noqa: F401
                         ut_inverse_rowloop, ut_inverse_solve)
from .l2norm import l2norm_rows  # noqa: F401
