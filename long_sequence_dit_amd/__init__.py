"""Long-sequence bidirectional attention for MI355X (gfx950).

The compute lives in ``libattn.so`` (HIP kernels behind the C ABI declared in
``include/attn.h``); ``long_sequence_dit_amd.attn`` is a thin ctypes binding
with the same entry-point names.  Importing this package loads nothing; the
binding loads the library on first use and fails loudly if it is missing.
"""

__all__ = ["attn"]
