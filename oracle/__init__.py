"""CPU oracle for the sparse decode step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy implementations of what the GPU path
computes, written from the pages (the Fathom summary, the OasisKV review and
the HashAttention study notes) and checked against closed forms, brute force
and the pages' worked example by the CPU test-suite.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The GPU library and its
Python binding never do: they share no code, header, table or helper with it.
The only thing both sides share is the seeded input generator (``synth``),
which holds no part of the method's arithmetic.

Precision: float64 for every real-valued result, except where a floating-point
comparison decides an integer (the 4-bit quantiser's codes and the read plan's
bit allocation); there the oracle computes in float32, the precision the GPU
path takes the same decision in.

Modules
  fathom   -- per-channel 4-bit quantiser, channel-major bit planes, the
              per-query reverse water-filling read plan, the plane-prefix scan
  select   -- top-k with lower-index tie-break and forced sink/local windows
  hamming  -- XOR/popcount signature distance
  quest    -- per-block min/max key summaries and their score
  attend   -- renormalised softmax attention over a selected set
"""
from . import fathom, select, hamming, quest, attend  # noqa: F401
