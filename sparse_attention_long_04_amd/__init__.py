"""MI355X-native DSA hot path: Lightning Indexer -> deterministic top-k -> sparse GQA attention.

The compute path is the C-ABI library ``libdsa.so`` (hand-written HIP for gfx950) declared in
``include/dsa.h``; :mod:`.dsa` is its thin ctypes binding.  Importing this package does not load
the library; the first call does, and raises if it is missing.
"""
