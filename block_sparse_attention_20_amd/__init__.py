"""Persistent Block-Sparse Attention (PBSA) for AMD Instinct MI355X.

The compute lives in ``libpbsa.so`` (hand-written HIP kernels for gfx950,
C ABI in ``include/pbsa.h``); this package is its Python binding
(``pbsa``), a per-layer buffer helper (``layer``) and the streaming rollout
driver (``rollout``).  Build with ``python -m block_sparse_attention_20_amd.build``.
"""
from . import pbsa  # noqa: F401
from .pbsa import PBSAError, lib  # noqa: F401
