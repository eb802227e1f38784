"""The allocation-free quantize entry point (sage_quantize_qk_noalloc) against sage_quantize_qk.

Both through the C ABI on the same inputs: every output (int8 codes, scales, K mean, LSE shift)
must be identical bit for bit.  Two calls in a row, the second on a smaller input, so that the
second reads none of the first call's partial sums left in the library's scratch array.  (Sizes
past the scratch array are refused by host validation: test_abi.py.)
"""

import ctypes

import numpy as np
import pytest
import torch

from quantized_attention_quantize_amd import api
from quantized_attention_quantize_amd.synthetic import make_inputs

from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu

def _outputs(g):
    return [g.q8, g.k8, g.q_scale, g.k_scale, g.k_mean, g.lse_corr]


def _run(L, q, k, noalloc):
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = api.alloc_quantized(B, H, Nq, Nk, d, q.device, Hkv=Hkv, dtype=q.dtype)
    for t in _outputs(g):
        t.fill_(-7 if t.dtype == torch.int8 else float("nan"))  # nothing left unwritten goes unnoticed
    dq, dk, st = api._desc(q, "HND"), api._desc(k, "HND"), g.cstruct()
    stream = api._stream(q)
    if noalloc:
        status = L.sage_quantize_qk_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(st), stream)
    else:
        ws = api.quantize_workspace(k.shape[0], Hkv, Nk, d, q.device)
        status = L.sage_quantize_qk(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(st), ws.data_ptr(), ws.numel(),
                                    stream)
    assert status == 0, api.load_library().sage_status_string(status)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in _outputs(g)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_noalloc_quantize_matches_workspace_entry(dtype):
    L = api.load_library()
    # the larger call first (B2 H8 Hkv4 N4000 d128), then a smaller one (B1 H2 N300 d64)
    for (B, H, Hkv, Nq, Nk, d, seed) in [(2, 8, 4, 3000, 4000, 128, 31), (1, 2, 2, 300, 300, 64, 32)]:
        say(f"no-alloc quantize B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype}")
        inp = make_inputs(B, H, Nq, Nk, d, sigma=4.0, seed=seed, Hkv=Hkv, dtype=dtype)
        q, k = inp.q.to(DEV), inp.k.to(DEV)
        want = _run(L, q, k, noalloc=False)
        got = _run(L, q, k, noalloc=True)
        for name, a, b in zip(["q8", "k8", "q_scale", "k_scale", "k_mean", "lse_corr"], got, want):
            assert a.shape == b.shape
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
