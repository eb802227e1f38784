"""Shared helpers of the GPU parity tests: moving seeded inputs to the device, undoing the
documented key order of the prepared V, and the comparison metrics."""

from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda"

from schedule import BLOCK_N, PLAIN_TOL, QE_TOL, ROW_TOL, ROWSUM_ROUNDED, TAU, TAU_FP4  # noqa: F401


def qe_schedule(pv: str) -> dict:
    """Keyword arguments of the oracle's emulation for the kernels' schedule."""
    return dict(BN=BLOCK_N, tau=TAU[pv], lsum_rounded=ROWSUM_ROUNDED)


def row_rel_l1(a, b) -> np.ndarray:
    """Per-row relative L1 of [R, d] arrays: sum_c |a - b| / sum_c |b| (0 for rows where both are
    all zero, inf where only b is)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.abs(a - b).sum(-1)
    den = np.abs(b).sum(-1)
    out = np.zeros(num.shape)
    nz = den > 0
    out[nz] = num[nz] / den[nz]
    out[~nz & (num > 0)] = np.inf
    return out


def check_o(got, want, pv: str, tag: str, plain=None) -> float:
    """O parity: aggregate relative L1 <= QE_TOL and every row within ROW_TOL[pv] of the emulation
    (want), and, when given, aggregate relative L1 <= PLAIN_TOL against the plain reading (plain).
    Returns the aggregate relative L1 against want."""
    e = rel_l1(got, want)
    rows = row_rel_l1(got, want)
    worst = float(rows.max()) if rows.size else 0.0
    msg = f"{tag}: rel-L1 vs emulation {e:.3e}, worst row {worst:.3e}"
    if plain is not None:
        ep = rel_l1(got, plain)
        msg += f", rel-L1 vs plain reading {ep:.3e}"
    say("  " + msg)
    assert e <= QE_TOL, msg
    assert worst <= ROW_TOL[pv], msg
    if plain is not None:
        assert ep <= PLAIN_TOL, msg
    return e


def say(*a):
    """Flushed progress line, so a failing GPU step names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp):
    return inp.q.to(DEV), inp.k.to(DEV), inp.v.to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32_of_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def fp16_storage_key(p: np.ndarray) -> np.ndarray:
    """Key held at storage position p of the prepared fp16 V (groups of 16: [0-3, 8-11, 4-7, 12-15])."""
    base = p & ~15
    q = p & 15
    return base + ((q & 7) >> 2) * 8 + (q >> 3) * 4 + (q & 3)


def fp8_storage_key(p: np.ndarray) -> np.ndarray:
    """Key held at storage position p of the prepared e4m3 V (groups of 64, see the header)."""
    base = p & ~63
    q = p & 63
    g, kb, r = q >> 5, (q >> 4) & 1, q & 15
    return base + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3)


def unpermute_vt(vt: np.ndarray, pv: str) -> np.ndarray:
    """[B,H,d,Nk_pad] in storage order -> [B,H,Nk_pad,d] in key order."""
    npad = vt.shape[-1]
    p = np.arange(npad)
    key = fp16_storage_key(p) if pv == "fp16" else fp8_storage_key(p)
    nat = np.empty_like(vt)
    nat[..., key] = vt
    return np.ascontiguousarray(np.swapaxes(nat, -1, -2))


def rel_l1(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).sum() / max(np.abs(b).sum(), 1e-300))


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def rows_of(out: torch.Tensor, rows: np.ndarray, layout: str = "HND") -> np.ndarray:
    """Pick flattened (b*H + h)*Nq + i rows of a [B,H,Nq,d] (or NHD) bf16 output as fp32."""
    o = out if layout == "HND" else out.permute(0, 2, 1, 3)
    B, H, Nq, d = o.shape
    flat = o.reshape(B * H * Nq, d) if o.is_contiguous() else o.contiguous().reshape(B * H * Nq, d)
    idx = torch.from_numpy(rows).to(out.device)
    return flat.index_select(0, idx).float().cpu().numpy()


def lse_rows(lse: torch.Tensor, rows: np.ndarray) -> np.ndarray:
    return lse.reshape(-1).index_select(0, torch.from_numpy(rows).to(lse.device)).cpu().numpy()


def assert_lse_close(got, want, atol):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), "LSE finiteness differs"
    assert np.array_equal(got[~fin], want[~fin])
    if fin.any():
        err = np.abs(got[fin] - want[fin]).max()
        assert err <= atol, f"LSE max abs diff {err} > {atol}"


def lse_quant_bound(qk, Qb, Kb, rows, Nq, Nk, sm_scale, causal=False, mask=None, dtype="bf16"):
    """Per-row bound on |LSE(quantized scores) - LSE(exact scores)|.

    logsumexp is 1-Lipschitz in the max norm, so the LSE moves by at most the largest score error
    over the row's visible keys.  With |q - qs*q8| <= qs/2 and |ks - ks*k8| <= ks/2 per element,
    |s_ij - s~_ij| <= sm * (sum_c |q_ic| * ks_j/2 + sum_c |k~_jc| * qs_i/2 + d * qs_i*ks_j/4),
    where k~ is the smoothed key (the smoothing shift itself cancels between the two LSEs, and so
    does an additive mask).  mask: uint8 (0 = masked) or float32 (-inf = masked); Qb, Kb are bits
    of ``dtype``."""
    B, H, _, d = Qb.shape
    grp = H // Kb.shape[1]  # query heads per key head (group-query attention)
    dec = f32_of_bf16_bits if dtype == "bf16" else (lambda b: b.view(np.float16).astype(np.float32))
    Q = dec(Qb).astype(np.float64)
    if qk.kmean.ndim == 4:  # per_block_mean: each key block smoothed by its own mean
        m = np.repeat(qk.kmean, 64, axis=2)[:, :, :Kb.shape[2]]
    else:
        m = qk.kmean[:, :, None, :]
    Ks = (dec(Kb) - m).astype(np.float32).astype(np.float64)
    sk = np.abs(Ks).sum(-1)  # [B,Hkv,Nk]
    out = np.empty(rows.size)
    for n, rid in enumerate(rows):
        bh, i = divmod(int(rid), Nq)
        b, h = divmod(bh, H)
        hk = h // grp
        qs = float(qk.qs[b, h, i // 64])
        ks = np.repeat(qk.ks[b, hk].astype(np.float64), 64)[:Nk]
        sq = np.abs(Q[b, h, i]).sum()
        bnd = sm_scale * (sq * ks / 2 + sk[b, hk] * qs / 2 + d * qs * ks / 4)
        valid = np.ones(Nk, bool)
        if causal:
            valid[i + 1:] = False
        if mask is not None:
            mrow = mask[b, 0 if mask.shape[1] == 1 else h, i]
            valid &= (mrow != -np.inf) if mask.dtype == np.float32 else (mrow != 0)
        out[n] = bnd[valid].max() if valid.any() else 0.0
    return out


# ---- FP4 microscaling method: undoing the documented packing and lane order of sage_fp4_qkv ----
def fp4_nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [..., n] pairs -> codes [..., 2n] (low nibble first)."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def fp4_qk_scales(sc: np.ndarray) -> np.ndarray:
    """lane-order scale bytes [..., d/32] -> logical blocks: block k sits at (k & 1) * (d/64) + k // 2."""
    nb = sc.shape[-1]
    pos = [(k & 1) * (nb // 2) + k // 2 for k in range(nb)]
    return sc[..., pos]


def fp4_v_scales(sc: np.ndarray, d: int) -> np.ndarray:
    """[..., nkb, d] lane order -> logical channel order: channel c at (c % 32) * (d/32) + c // 32."""
    pos = [(c % 32) * (d // 32) + c // 32 for c in range(d)]
    return sc[..., pos]


def fp4_check_quant(g, r, Nq, Nk, vq=None, k_max=1.0):
    """GPU packed buffers against the oracle's FP4QK (r) and V codes (vq = (v4, ve)); k_max bounds
    |K| and |K - kmean| (for the correction rows' fp32 accumulation bound)."""
    q4 = fp4_nibbles(g.q4.cpu().numpy())
    k4 = fp4_nibbles(g.k4.cpu().numpy())
    assert np.array_equal(g.k_mean.cpu().numpy(), r.kmean), "k_mean"
    assert np.array_equal(g.q_mean.cpu().numpy(), r.qmean), "q_mean"
    assert np.array_equal(q4[:, :, :Nq], r.q4), "q codes"
    assert np.array_equal(k4[:, :, :Nk], r.k4), "k codes"
    assert not q4[:, :, Nq:].any() and not k4[:, :, Nk:].any(), "pad rows"
    assert np.array_equal(fp4_qk_scales(g.q_scale.cpu().numpy())[:, :, :Nq], r.qe), "q scales"
    assert np.array_equal(fp4_qk_scales(g.k_scale.cpu().numpy())[:, :, :Nk], r.ke), "k scales"
    np.testing.assert_allclose(g.lse_corr.cpu().numpy(), r.lse_corr, rtol=2e-6, atol=2e-6)
    corr = g.qk_corr.cpu().numpy()
    # the GPU sums exact products qmean_c K_jc in fp32 from -(qmean . kmean): its error stays well
    # inside 1e-5 of sum_c |qmean_c| max(|K_jc|, |kmean_c|)
    bound = np.abs(r.qmean).max() * k_max * r.qmean.shape[-1]
    np.testing.assert_allclose(corr[..., :Nk], r.qk_corr, rtol=0, atol=1e-5 * bound + 1e-30)
    assert not corr[..., Nk:].any()
    if vq is not None:
        v4, ve = vq
        vt = fp4_nibbles(g.v4t.cpu().numpy())  # [B, Hkv, d, Nk_pad]
        assert np.array_equal(np.swapaxes(vt, -1, -2)[:, :, :Nk], v4), "v codes"
        assert not vt[..., Nk:].any()
        nkb = ve.shape[2]
        assert np.array_equal(fp4_v_scales(g.v_scale.cpu().numpy(), v4.shape[-1])[:, :, :nkb], ve), "v scales"
