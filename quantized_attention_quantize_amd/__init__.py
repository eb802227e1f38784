"""MI355X-native SageAttention-style quantized attention forward (INT8 QK, FP16/FP8 PV; MX FP4).

The compute path is a C-ABI shared library of hand-written gfx950 HIP kernels
(``libsage_mi355x.so``, built from ``csrc/``); this package is a thin ctypes binding over it.
PyTorch supplies device memory and the current stream only.  Importing the package does not load
the library; the first call does, and raises if the library is missing.
"""

from .api import (  # noqa: F401
    SageError,
    attn_fwd,
    attn_fwd_prepared,
    block_n,
    debug_qk_int32,
    lib_path,
    load_library,
    merge_lse,
    pad_tokens,
    prepare_v,
    quantize_qk,
    quantize_qk_varlen,
    rowsum_rounded,
    sageattn,
    sageattn_varlen,
    softmax_tau,
)
from .fp4 import (  # noqa: F401
    QuantizedFP4,
    attn_fwd_fp4,
    debug_scores_fp4,
    quantize_qkv_fp4,
    sageattn_fp4,
    softmax_tau_fp4,
)
