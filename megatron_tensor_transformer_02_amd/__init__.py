"""MI355X-native tensor-parallel transformer-layer shard library.

The compute path is ``libmp.so`` (hand-written HIP for gfx950 behind the C ABI
declared in ``include/mp.h``); :mod:`.mp` is its thin ctypes binding and
:mod:`.synthetic` draws the seeded inputs.  Importing this package loads
nothing; the library is opened on first use and a missing library is an
error, never a fallback.
"""

__all__ = ["mp", "synthetic"]
