"""MI355X (gfx950) sparse top-k decode query: bit-plane / signature / block
summary scoring, top-k selection and gather attention in hand-written HIP.

The compute path is the C-ABI library ``libsdq.so`` built from ``csrc/``
(declared in ``include/sdq.h``); ``sparse_top_decode_query_amd.lib`` is its
thin ctypes binding.  Importing the package does not load the library; the
first call into ``lib`` does, and raises if it has not been built.
"""
from . import bytemodel, lib  # noqa: F401

__all__ = ["lib", "bytemodel"]
