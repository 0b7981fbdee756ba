"""CPU oracle (test infrastructure only).

Plain, slow, float64 implementations of what the decoder block computes
(``ref``: vectorised numpy; ``brute``: scalar loops for tiny shapes).  Only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package; the library under ``decoder_block_rmsnorm_amd`` never
does, and this package imports nothing from it.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` to
closed forms, invariants, library routines (torch's scaled_dot_product_attention
and silu on the CPU) and the brute-force loops.  End-to-end block outputs are
pinned only through those pieces and their composition: the pages print no
worked numeric example of a block output.
"""
from . import ref, brute  # noqa: F401
