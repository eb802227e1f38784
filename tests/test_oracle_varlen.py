"""Pins for the oracle's packed variable-length batches (docs digest, ``sageattn_varlen``).

Exact attention one sequence at a time equals exact attention over the whole packed batch under a
block-diagonal mask (causal: each block lower-triangular from its own first query and key), a
structure written here independently of the oracle.  The quantized emulation of equal-length
sequences equals the dense batched emulation with one batch entry per sequence; empty sequences
change nothing else; a sequence without keys gives O = 0 and LSE = -inf.
"""

import numpy as np
import pytest

from quantized_attention_quantize_amd.synthetic import make_varlen_inputs


def _to_dense_hnd(X):
    """packed [T, H, d] -> [1, H, T, d]"""
    return np.ascontiguousarray(np.transpose(X, (1, 0, 2))[None])


def _block_diag_mask(cu_q, cu_k, causal):
    cu_q, cu_k = list(cu_q), list(cu_k)
    m = np.zeros((1, 1, cu_q[-1], cu_k[-1]), np.uint8)
    for b in range(len(cu_q) - 1):
        nq, nk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        blk = np.ones((nq, nk), np.uint8)
        if causal:
            blk = np.tril(blk)  # key j visible to query i iff j <= i, both counted from the sequence start
        m[0, 0, cu_q[b]:cu_q[b + 1], cu_k[b]:cu_k[b + 1]] = blk
    return m


@pytest.mark.parametrize("causal", [False, True])
def test_exact_varlen_is_block_diagonal_attention(orc, causal):
    sq, sk = [70, 1, 130, 64], [90, 5, 130, 33]
    inp = make_varlen_inputs(sq, sk, 2, 64, seed=50)
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    o, l = orc.attn_ex_varlen(Q, K, V, inp.cu_q.tolist(), inp.cu_k.tolist(), causal=causal)
    m = _block_diag_mask(inp.cu_q.tolist(), inp.cu_k.tolist(), causal)
    do, dl = orc.attn_ex(_to_dense_hnd(Q), _to_dense_hnd(K), _to_dense_hnd(V), mask=m)
    H, T, d = 2, sum(sq), 64
    np.testing.assert_allclose(o, do.reshape(H, T, d).transpose(1, 0, 2), rtol=0, atol=1e-12)
    fin = np.isfinite(dl.reshape(H, T))
    assert np.array_equal(np.isfinite(l), fin)
    np.testing.assert_allclose(l[fin], dl.reshape(H, T)[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("pv,causal", [("fp16", False), ("fp8", True)])
def test_equal_lengths_equal_dense_batch(orc, pv, causal):
    nseq, n, H, d = 3, 96, 2, 128
    inp = make_varlen_inputs([n] * nseq, [n] * nseq, H, d, seed=51, sigma=4.0 if pv == "fp16" else 8.0)
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    o32, o16, lse = orc.run_qe_varlen(Q, K, V, inp.cu_q.tolist(), inp.cu_k.tolist(), pv=pv, causal=causal)

    def dense(X):  # [nseq*n, H, d] -> [nseq, H, n, d]
        return np.ascontiguousarray(X.reshape(nseq, n, H, d).transpose(0, 2, 1, 3))

    r = orc.run_qe(dense(Q), dense(K), dense(V), pv=pv, causal=causal)
    assert np.array_equal(o32, r.o32.reshape(nseq, H, n, d).transpose(0, 2, 1, 3).reshape(nseq * n, H, d))
    assert np.array_equal(lse, r.lse.reshape(nseq, H, n).transpose(1, 0, 2).reshape(H, nseq * n))


def test_empty_sequences_and_keyless_rows(orc):
    inp = make_varlen_inputs([50, 0, 40, 30], [60, 20, 45, 0], 2, 64, seed=52)
    Q, K, V = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    o32, o16, lse = orc.run_qe_varlen(Q, K, V, inp.cu_q.tolist(), inp.cu_k.tolist())
    # the last sequence has queries but no keys
    assert (o32[90:] == 0).all() and np.isneginf(lse[:, 90:]).all()
    # dropping the empty-query sequence (its keys are never seen) leaves the others unchanged
    keep_k = np.concatenate([np.arange(0, 60), np.arange(80, 125)])
    o2, _, l2 = orc.run_qe_varlen(Q[:90], K[keep_k], V[keep_k], [0, 50, 90], [0, 60, 105])
    assert np.array_equal(o32[:90], o2) and np.array_equal(lse[:, :90], l2)
