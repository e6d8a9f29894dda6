"""MI355X-native Mamba-2 SSD layer hot path.

The compute lives in libssd.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/ssd.h); `state_space_sequence_ssd_amd.ssd` is the thin ctypes
binding with the same entry-point names.  Importing this package loads
nothing; the library is loaded on the first call.
"""
__all__ = ["inputs", "ssd"]
