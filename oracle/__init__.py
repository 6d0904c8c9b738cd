"""fp64 CPU oracle of Persistent Block-Sparse Attention (PBSA).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It is written from the
method's description (see the module docstrings for the pages and sections)
and shares no code with the HIP path.

Parity status of each function is recorded next to its pins in
``tests/test_oracle_pins.py``; the readings R2-R5, R11-R13, R15 that the
pages leave open cannot be pinned by the pages themselves ("parity unpinned"
for those readings; only self-consistency and arithmetic checks apply).
"""
from . import pbsa_oracle, rollout  # noqa: F401
