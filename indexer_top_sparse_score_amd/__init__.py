"""MI355X (gfx950) indexer -> Top-K -> sparse-attention decode step.

The compute lives in libdsa.so (hand-written HIP, C ABI in include/dsa.h);
``binding`` is its ctypes wrapper.  Build the library with
``python -m indexer_top_sparse_score_amd.build``.
"""

from . import binding  # noqa: F401

__all__ = ["binding"]
