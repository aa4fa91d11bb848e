"""Occult MoE layer on AMD MI355X (gfx950): HIP kernels behind a C ABI.

The compute lives in ``libocc.so`` (sources in ``csrc/``, ABI in
``include/occ.h``); ``occ`` is its thin ctypes binding.  Submodules are
imported on demand so that the seeded input generator can be used without
loading the library.
"""
