"""Where a non-finite input may show up in the outputs: the reach sets of the library's NaN policy,
written from the policy's statement alone (no oracle, no kernel), shared by the oracle's pins and
the GPU tests.

The policy: a NaN (or an infinity that the arithmetic turns into one) is never dropped and never
becomes a finite value.
  * A quantization group's scale is NaN when the group holds a NaN: the 64-token blocks of Q and
    of smoothed K, and an FP8 V channel.  Every code of such a group is 0.  Means (K's per-head
    or per-block mean, V's mean under smooth_v) are plain sums, NaN when a summand is.
  * A row's O and LSE are NaN when one of its visible keys has a NaN score: its Q block's scale,
    the scale or mean of the key's K block, or K's per-head mean is NaN.  A row without a visible
    key gives O = 0 and LSE = -inf whatever the inputs hold.
  * A NaN in fp16 V at (key j, channel c) reaches O[i, c] for every row i with a visible key whose
    key loop covers j's 64-key tile (a zero probability times NaN is NaN).  Rows that see key j
    are always reached; which others are depends on the key loop (``loop``): "oracle" -- under
    causal masking a row's loop ends at the last tile holding one of its keys; "kernel" -- the
    loop of the row's 256-row block: under causal masking the tiles up to that block's last row,
    and tiles entirely masked for the block are skipped.  An NaN FP8 V channel scale or smooth_v
    channel mean reaches channel c of every row with a visible key.  V never reaches the LSE.
"""

from __future__ import annotations

import numpy as np

QBLK = 64  # tokens per quantization block
BN = 64  # keys per tile
BM = 256  # query rows per block of the GPU key loop


def visible(Nq: int, Nk: int, causal: bool, mask=None) -> np.ndarray:
    """bool [Nq, Nk]: key j is visible to row i (mask: bool [Nq, Nk], True = attend, or None)."""
    vis = np.ones((Nq, Nk), bool)
    if causal:
        vis &= np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    if mask is not None:
        vis &= np.asarray(mask, bool)
    return vis


def live_rows(vis: np.ndarray) -> np.ndarray:
    return vis.any(1)


def reach_q(vis: np.ndarray, i0: int) -> np.ndarray:
    """Rows (bool [Nq]) whose O and LSE a NaN in Q row i0 makes NaN: its quantization block's."""
    blk = np.arange(vis.shape[0]) // QBLK == i0 // QBLK
    return blk & live_rows(vis)


def reach_k_head(vis: np.ndarray) -> np.ndarray:
    """Rows made NaN by a NaN in K under per-head smoothing: every row with a visible key."""
    return live_rows(vis)


def reach_k_block(vis: np.ndarray, j0: int) -> np.ndarray:
    """Rows made NaN by a NaN in K key j0 when K blocks are smoothed by their own means: the rows
    that see a key of j0's block."""
    u = j0 // QBLK
    return vis[:, u * QBLK:(u + 1) * QBLK].any(1)


def covers_tile(Nq: int, Nk: int, causal: bool, u: int, loop: str, mask=None) -> np.ndarray:
    """bool [Nq]: the key loop of row i covers tile u."""
    i = np.arange(Nq)
    if loop == "oracle":
        return i >= u * BN if causal else np.ones(Nq, bool)
    assert loop == "kernel"
    qt = i // BM
    nkt = -(-Nk // BN)
    kt_end = np.minimum(nkt, (qt * BM + BM + BN - 1) // BN) if causal else np.full(Nq, nkt)
    cov = u < kt_end
    if mask is not None:
        m = np.asarray(mask, bool)[:, u * BN:(u + 1) * BN]
        for b in range(-(-Nq // BM)):
            if not m[b * BM:(b + 1) * BM].any():
                cov[b * BM:(b + 1) * BM] = False
    return cov


def reach_v16(vis: np.ndarray, j0: int, causal: bool, loop: str, mask=None) -> np.ndarray:
    """Rows whose channel c a NaN in fp16 V at (j0, c) makes NaN."""
    Nq, Nk = vis.shape
    return covers_tile(Nq, Nk, causal, j0 // BN, loop, mask) & live_rows(vis)


def must_v(vis: np.ndarray, j0: int) -> np.ndarray:
    """Rows that see key j0: reached under any key loop."""
    return vis[:, j0].copy()
