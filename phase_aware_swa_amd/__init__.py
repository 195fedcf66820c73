"""MI355X-native Orthros phase-aware heterogeneous attention (one layer).

The compute path is the C-ABI library ``liborthros.so`` built from
``csrc/`` (hand-written HIP for gfx950); ``binding`` is its thin ctypes
wrapper.  Importing this package does not load the library: the first call
through ``binding`` does, and fails loudly when it is not built.
"""
