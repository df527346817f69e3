"""Exact tiled attention on AMD Instinct MI355X (gfx950).

The compute lives in a C-ABI shared library built from ``csrc/`` (hand-written
HIP kernels); :mod:`.attn` is a thin ctypes binding over it.  Importing the
package does not load the library; the first call through :mod:`.attn` does,
and fails loudly if it has not been built.
"""

__all__ = ["attn", "workloads"]
