"""MI355X-native MoE decode hot path: 4-bit affine expert GEMVs, int8 router with top-k, combine with the
shared expert, and a per-layer LFU expert cache — HIP kernels for gfx950 behind the C ABI in
``include/moeq4.h`` (``libmoeq4.so``), with a thin ctypes binding in ``moeq4``.
"""
