"""MI355X-native SageAttention-style quantized attention forward (INT8 QK, FP16/FP8 PV).

The compute path is a C-ABI shared library of hand-written gfx950 HIP kernels
(``libsage_mi355x.so``, built from ``csrc/``); this package is a thin ctypes binding over it.
PyTorch supplies device memory and the current stream only.
"""
