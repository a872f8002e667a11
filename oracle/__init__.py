"""CPU oracle for the packed ternary-hybrid matrix-vector product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (no kernels, headers, helpers, tables or constants); the two meet
only through the seeded input generator in ``synth``.

What it computes is the operator printed on the WAL-Ternary-8B model pages
(Kazakh card, section "Модель пішімі"; English card, section
"Representation"):

    W(x) = (alpha * T + beta * R) x + sum_r U_r (V_r^T x)

with the per-128-group scales of the WAL2-Ternary-27B card (section
"Архитектура": scale group 128) and the two binary paths and 24-bit scales of
the WAL-Ternary-27B-RC1 card (section "Representation").  It does so in the
plainest way: decode the packed blob with an independent numpy decoder into
the logical arrays, build the dense float64 matrix W, and multiply.

Modules:
  ``oracle.format`` - independent numpy packer, unpacker, validator, sizes.
  ``oracle.dense``  - dense float64 W and products y = W x, Y = X W^T.
  ``oracle.rotation`` - the normalised Hadamard-128 rotation of x (the
                        WAL2-Ternary-27B card's rotation, "Архитектура").
  ``oracle.int4``   - INT4/g128 packed matrices (the 8B cards' LM head).
  ``oracle.int3``   - INT3/g128 packed matrices and embedding rows (the 8B
                      cards' embedding).
  ``oracle.int5``   - INT5/g128 packed matrices (the RC1 card's LM head).

Every function is pinned by tests under ``tests/`` against facts other than
itself (golden bytes worked from the format readings, byte totals printed on
the pages, exact-rational brute force, library special cases, invariants).
"""
from . import format, dense, rotation, int4, int3, int5  # noqa: F401
