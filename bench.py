#!/usr/bin/env python
"""Throughput of the quantized attention forward on one MI355X.

One step = the whole hot path on one batch of seeded synthetic input already resident in HBM:
sage_quantize_qk (K mean, INT8 Q/K, scales, LSE shift) -> sage_prepare_v (fp16 or e4m3 V) ->
sage_attn_fwd_prepared (mask classification if any, attention with LSE).

    python bench.py [--steps K] [--warmup W] [--workload n8k]

Prints one JSON line.  ``value`` is attention TOPS = 4*B*H*Nq*Nk*d / (time per step), halved for
causal, over the whole step.  ``roofline`` reports the attention kernel alone: its algorithmic
ops per launch over its average duration, measured with HIP events recorded on the stream the
kernel runs on, against the MFMA peak of its own dtypes (INT8 for QK^T, FP16 or FP8 for PV).  ``cpu_baseline`` times the CPU oracle (the
plain reference implementation used by the tests) on a bounded sample of the same workload.

The FP4 workloads (``fp4_b1h24n4096``, ``n8k_fp4``) time the FP4 microscaling method instead:
sage_fp4_quantize_qkv (smoothing, MX FP4 Q/K/V, correction rows) -> sage_fp4_attn_fwd, with the
roofline of k_fp4_attn against the FP4 (QK^T) and FP8 (PV) MFMA peaks.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TOPS (4·B·H·N²·d/t) and % of dense INT8 MFMA peak, 1×MI355X"
INT8_PEAK_TOPS = 5000.0  # MI355X dense INT8 MFMA (datasheet, no sparsity); FP8 is the same
FP16_PEAK_TOPS = 2500.0  # MI355X dense FP16 MFMA


FP4_PEAK_TOPS = 10100.0  # MI355X dense FP4 MFMA
SETTLE_S = 0.25  # seconds of back-to-back untimed steps before the timed region (see run_timed)
FP8_PEAK_TOPS = 5000.0


def mfma_peak(pv: str, method: str = "int8") -> float:
    """MFMA ceiling of the attention kernel for its own dtypes: half its counted ops are QK^T (INT8,
    or e2m1 for the FP4 method), half are PV (FP16, FP8, or e2m1 x e4m3 at the FP8 rate), so the
    ceiling is the harmonic combination of the two peaks."""
    if method == "fp4":
        return 1.0 / (0.5 / FP4_PEAK_TOPS + 0.5 / FP8_PEAK_TOPS)
    pv_peak = FP16_PEAK_TOPS if pv == "fp16" else INT8_PEAK_TOPS
    return 1.0 / (0.5 / INT8_PEAK_TOPS + 0.5 / pv_peak)
KERNEL_SOURCES = {"k_attn_fwd": ["quantized_attention_quantize_amd/csrc/sage_attn.hip",
                                  "quantized_attention_quantize_amd/csrc/sage_device.h",
                                  "quantized_attention_quantize_amd/csrc/sage_launch.h"],
                  "k_fp4_attn": ["quantized_attention_quantize_amd/csrc/sage_fp4.hip",
                                 "quantized_attention_quantize_amd/csrc/sage_device.h"]}


def kernel_source_hash(kernel: str = "k_attn_fwd") -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _profile(name: str, kernel: str):
    """A committed profile summary (profiles/<name>.json) if it was taken on the current kernel
    source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("kernel_source_hash") == kernel_source_hash(kernel) else None


def traffic_from_profile(workload: str, kernel: str = "k_attn_fwd"):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    t = _profile(f"{kernel}_{workload}_hbm_traffic", kernel)
    return None if t is None else t.get("bytes_per_launch")


def valu_ceiling(workload: str, ops_per_launch: float, kernel: str = "k_attn_fwd"):
    """The VALU ceiling of the attention kernel: its own vector-ALU instructions per launch (the
    committed rocprofv3 counts SQ_INSTS_VALU minus SQ_INSTS_MFMA, split into transcendental
    (SQ_INSTS_VALU_TRANS_F32), conversion (SQ_INSTS_VALU_CVT) and the rest) times the measured time
    each takes on one SIMD at full occupancy (profiles/isa_rates_gfx950.json: v_exp_f32,
    v_cvt_f32_i32, v_fma_f32), spread over every SIMD.  The rate at which these instructions could
    complete if nothing else limited the kernel, as ops/s; None without a profile of the current
    kernel source."""
    c = _profile(f"{kernel}_{workload}_counters", kernel)
    rates_path = os.path.join(ROOT, "profiles", "isa_rates_gfx950.json")
    if c is None or not os.path.exists(rates_path):
        return None
    with open(rates_path) as f:
        r = json.load(f)["ns_per_wave_instr_per_simd_8wps"]
    per = c["per_dispatch"]
    trans, cvt = per["SQ_INSTS_VALU_TRANS_F32"], per["SQ_INSTS_VALU_CVT"]
    other = per["SQ_INSTS_VALU"] - per["SQ_INSTS_MFMA"] - trans - cvt
    simds = 4 * c["cus"]
    ns = (trans * r["v_exp_f32"] + cvt * r["v_cvt_f32_i32"] + other * r["v_fma_f32"]) / simds
    return {"peak": round(ops_per_launch / (ns * 1e-9) / 1e12, 1), "unit": "TOPS", "ms": round(ns * 1e-6, 4),
            "valu_instr_per_launch": {"transcendental": trans, "conversion": cvt, "other": other},
            "basis": "the kernel's VALU instructions per launch (rocprofv3 counts) x measured ns per "
                     "instruction per SIMD at 8 waves/SIMD (bench_isa_rates.hip), over 1024 SIMDs"}


def _read_sclk(paths):
    """Current shader clock(s) in MHz from the sysfs DPM tables (the line marked '*')."""
    import re

    mhz = []
    for p in paths:
        try:
            for ln in open(p):
                if ln.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", ln, flags=re.I)
                    if m:
                        mhz.append(int(m.group(1)))
        except OSError:
            pass
    return mhz


def _amdsmi_gfx_clocks():
    """Current GFX clock of every XCD (MHz) from amd-smi: the CLK lines of the GFX_n sections only."""
    import re
    import subprocess

    r = subprocess.run(["amd-smi", "metric", "-c", "-g", "0"], capture_output=True, text=True, timeout=5)
    mhz, in_gfx = [], False
    for ln in r.stdout.splitlines():
        sec = re.match(r"^\s+([A-Z]+)_\d+:\s*$", ln)
        if sec:
            in_gfx = sec.group(1) == "GFX"
            continue
        m = re.match(r"^\s+CLK:\s+(\d+) MHz", ln)
        if m and in_gfx:
            mhz.append(int(m.group(1)))
    return mhz


def sample_clocks(out_path: str, stop_path: str):
    """--sample-clocks: write the shader clock (MHz) with a timestamp every 5 ms (sysfs pp_dpm_sclk;
    amd-smi's GFX clocks every 0.1 s where sysfs has none) until stop_path exists.  Started by the
    benchmark before it touches the GPU."""
    import glob

    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    parent, t_end = os.getppid(), time.time() + 1800
    with open(out_path, "w") as out:
        # until told to stop, or the benchmark process is gone, or half an hour has passed
        while not os.path.exists(stop_path) and os.getppid() == parent and time.time() < t_end:
            t = time.time()
            try:
                mhz = _read_sclk(paths) if paths else _amdsmi_gfx_clocks()
            except Exception:
                mhz = []
            out.write(json.dumps({"t": t, "mhz": mhz}) + "\n")
            out.flush()
            time.sleep(0.005 if paths else 0.1)


def start_clock_sampler():
    """Starts the clock sampler in a child process before any GPU use; returns a function that stops
    it and gives the GFX clock readings (MHz) taken between two wall-clock times."""
    import subprocess
    import tempfile

    d = tempfile.mkdtemp(prefix="sage_clk_")
    out, stop = os.path.join(d, "clk.jsonl"), os.path.join(d, "stop")
    try:
        p = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--sample-clocks", out, stop],
                             stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    except Exception:
        return lambda t0, t1: None

    def finish(t0, t1):
        open(stop, "w").close()
        try:
            p.wait(timeout=10)
        except Exception:
            p.kill()
        mhz = []
        if os.path.exists(out):
            for line in open(out):
                rec = json.loads(line)
                if t0 <= rec["t"] <= t1:
                    mhz += [m for m in rec["mhz"] if m > 0]
        if not mhz:
            return None
        mhz.sort()
        return {"median_mhz": mhz[len(mhz) // 2], "min_mhz": mhz[0], "max_mhz": mhz[-1], "readings": len(mhz),
                "source": "current shader clock (sysfs pp_dpm_sclk, else amd-smi GFX clocks), sampled every "
                          "5 ms during the timed steps"}

    return finish


def accuracy_rows(q, k, v, out, causal: bool, mask, heads: int = 2, rows_per_head: int = 128, seed: int = 7):
    """Output accuracy on sampled rows against plain PyTorch fp32 attention on the same bf16/fp16
    inputs (exact softmax, no quantization), computed on the GPU after the timed steps.  q, out:
    [B, H, Nq, d]; k, v: [B, Hkv, Nk, d]; mask: None or broadcastable [B, 1|H, Nq, Nk] (bool: True
    attends; float: added)."""
    import torch

    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = torch.Generator().manual_seed(seed)
    sm = 1.0 / (d ** 0.5)
    num = den = dot = nq = no = 0.0
    worst = 0.0
    n = 0
    for hh in torch.randperm(B * H, generator=g)[:heads].tolist():
        b, h = divmod(hh, H)
        hk = h // (H // Hkv)
        rows = torch.randperm(Nq, generator=g)[:rows_per_head].sort().values.to(q.device)
        qr = q[b, h].index_select(0, rows).float()
        kt = k[b, hk].float().t().contiguous()
        s = (qr @ kt) * sm
        if causal:
            s = s.masked_fill(torch.arange(Nk, device=q.device)[None, :] > rows[:, None], float("-inf"))
        if mask is not None:
            m = mask[b, 0 if mask.shape[1] == 1 else h]
            m = m.expand(Nq, Nk) if m.shape[0] == 1 else m
            m = m.index_select(0, rows)
            s = s.masked_fill(~m, float("-inf")) if m.dtype == torch.bool else s + m.float()
        p = torch.softmax(s, dim=-1).nan_to_num(0.0)
        ref = p @ v[b, hk].float()
        got = out[b, h].index_select(0, rows).float()
        err = (got - ref).abs().sum(-1)
        mag = ref.abs().sum(-1)
        num += float(err.sum())
        den += float(mag.sum())
        worst = max(worst, float((err / mag.clamp_min(1e-30)).max()))
        dot += float((got * ref).sum())
        nq += float((got * got).sum())
        no += float((ref * ref).sum())
        n += int(rows.numel())
    return {"rows": n, "rel_l1_vs_fp32": round(num / max(den, 1e-300), 6), "worst_row_rel_l1": round(worst, 6),
            "cosine": round(dot / max((nq * no) ** 0.5, 1e-300), 6),
            "reference": "plain PyTorch fp32 softmax attention on the same inputs, sampled rows of the last step"}


def cpu_baseline(w, work_target: float, tau: float, lsum_rounded: bool):
    """The oracle (never tuned) on a bounded sample of the workload: whole heads (B=1) of the same
    shape and input recipe -- K mean, INT8 quantization and V preparation of those heads, then the
    quantized emulation of evenly spaced query rows -- sized to about `work_target` row x key
    pairs (~15 s on 16 host cores at the default)."""
    import math

    import numpy as np
    import torch

    import oracle
    from quantized_attention_quantize_amd.synthetic import make_inputs

    oracle.build(force=False)
    if w.method == "fp4":  # its emulation dequantizes every product in fp64: about 3x the INT8 cost per pair
        work_target /= 3.0
    if w.seqlens:  # a packed batch: sample whole heads of its first sequence
        import dataclasses
        w = dataclasses.replace(w, B=1, Nq=w.seqlens[0], Nk=w.seqlens[0], seqlens=())
    heads = max(1, min(w.B * w.H, math.ceil(work_target / (w.Nq * w.Nk))))
    per_head = max(1, min(w.Nq, int(work_target / (heads * w.Nk))))
    g = w.H // (w.Hkv or w.H)  # query heads per key/value head
    inp = make_inputs(1, heads, w.Nq, w.Nk, w.d, w.sigma, seed=0, mask=w.mask,
                      Hkv=max(1, heads // g) if g > 1 and heads % g == 0 else 0,
                      dtype=torch.float16 if w.dtype == "fp16" else torch.bfloat16)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    local = np.linspace(0, w.Nq - 1, per_head).astype(np.int64)
    rows = np.concatenate([h * w.Nq + local for h in range(heads)])
    if w.method == "fp4":
        t0 = time.perf_counter()
        oracle.run_fp4(Qb, Kb, Vb, causal=w.causal, per_block_mean=w.per_block_mean, tau=tau, rows=rows,
                       dtype=w.dtype)
        dt = time.perf_counter() - t0
        ops = 4.0 * rows.size * w.Nk * w.d / (2 if w.causal else 1)
        return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": f"{heads} head(s) (B=1) of {w.name}: smoothing and MX FP4 quantization of the heads' Q, K "
                          f"and V, FP4 emulation of {per_head} evenly spaced query rows per head x {w.Nk} keys; "
                          f"{dt:.2f} s"}
    t0 = time.perf_counter()
    S = w.kv_splits
    bounds = [w.Nk * s // S for s in range(S + 1)]
    parts = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):  # one slice, or all keys
        Ks, Vs = np.ascontiguousarray(Kb[:, :, lo:hi]), np.ascontiguousarray(Vb[:, :, lo:hi])
        qk = oracle.quant_qk(Qb, Ks, dtype=w.dtype, per_block_mean=w.per_block_mean)
        vm = oracle.kmean(Vs, w.dtype) if w.smooth_v else None
        vh, vs = oracle.prep_v(Vs, w.pv, dtype=w.dtype, vmean=vm)
        parts.append(oracle.attn_qe(qk, vh, vs, w.pv, w.Nq, hi - lo, causal=w.causal, mask=inp.mask_u8, BN=64,
                                    tau=tau, lsum_rounded=lsum_rounded, rows=rows, out_dtype=w.dtype, vmean=vm))
    if S > 1:
        oracle.merge_lse(np.stack([p[0] for p in parts]), np.stack([p[2] for p in parts]))
    dt = time.perf_counter() - t0
    if w.causal:
        ops = heads * float(sum(4.0 * (int(i) + 1) * w.d for i in local))
    else:  # the mask workload counts formula ops too, as the GPU metric does
        ops = 4.0 * rows.size * w.Nk * w.d
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{heads} head(s) (B=1) of {w.name}: K mean + INT8 quantization + V prep of the heads"
                      f"{f' per key slice ({S}), merged' if S > 1 else ''}, "
                      f"quantized emulation of {per_head} evenly spaced query rows per head x {w.Nk} keys; "
                      f"{dt:.2f} s"}


def varlen_setup(w, dev):
    """Packed variable-length workload: buffers allocated once; step = per-sequence K mean and INT8
    quantization, V preparation, attention (one launch over all sequences)."""
    import torch

    from quantized_attention_quantize_amd import api
    from quantized_attention_quantize_amd.synthetic import make_varlen_inputs

    vin = make_varlen_inputs(list(w.seqlens), list(w.seqlens), w.H, w.d, w.sigma, seed=0, Hkv=w.Hkv,
                             dtype=torch.float16 if w.dtype == "fp16" else torch.bfloat16)
    q, k, v = vin.q.to(dev), vin.k.to(dev), vin.v.to(dev)
    cq, ck = vin.cu_q.to(dev), vin.cu_k.to(dev)
    nseq, mx, Hkv = len(w.seqlens), max(w.seqlens), w.Hkv or w.H
    qk = api.alloc_quantized(nseq, w.H, mx, mx, w.d, dev, Hkv=Hkv, dtype=q.dtype)
    qws = api.quantize_workspace(nseq, Hkv, mx, w.d, dev)
    vt_vs = api.alloc_prepared_v(nseq, Hkv, mx, w.d, w.pv, dev)
    vws = api.prepare_v_workspace(nseq, Hkv, mx, w.d, w.pv, dev)
    out = torch.empty_like(q)
    lse = torch.empty(w.H, q.shape[0], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None, mev=None):
        api.quantize_qk_varlen(q, k, cq, ck, mx, mx, out=qk, workspace=qws)
        api.prepare_v_varlen(v, ck, mx, w.pv, out=vt_vs, workspace=vws)
        if ev is not None:
            ev[0][0].record(stream)
        api.attn_fwd_prepared_varlen(qk, vt_vs[0], vt_vs[1], cq, ck, q.shape[0], k.shape[0], pv_dtype=w.pv,
                                     is_causal=w.causal, return_lse=w.lse, out=out, lse=lse if w.lse else None)
        if ev is not None:
            ev[0][1].record(stream)

    def accuracy():  # the first sequence of the packed batch
        n0 = w.seqlens[0]
        hnd = lambda x: x[:n0].permute(1, 0, 2).unsqueeze(0)  # noqa: E731
        return accuracy_rows(hnd(q), hnd(k), hnd(v), hnd(out), w.causal, None)

    return step, 1, out.element_size(), accuracy


def fp4_setup(w, dev):
    """FP4 microscaling workload: buffers allocated once; step = smoothing and MX FP4 quantization of
    Q, K, V with the correction rows, then attention."""
    import torch

    from quantized_attention_quantize_amd import fp4
    from quantized_attention_quantize_amd.synthetic import workload_inputs

    inp = workload_inputs(w, seed=0)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    del inp
    Hkv = w.Hkv or w.H
    qkv = fp4.alloc_fp4(w.B, w.H, Hkv, w.Nq, w.Nk, w.d, dev, per_block_mean=w.per_block_mean, dtype=q.dtype)
    ws = fp4.fp4_workspace(w.B, w.H, Hkv, w.Nq, w.Nk, w.d, dev)
    out = torch.empty(w.B, w.H, w.Nq, w.d, dtype=q.dtype, device=dev)
    lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None, mev=None):
        fp4.quantize_qkv_fp4(q, k, v, per_block_mean=w.per_block_mean, out=qkv, workspace=ws)
        if ev is not None:
            ev[0][0].record(stream)
        fp4.attn_fwd_fp4(qkv, is_causal=w.causal, return_lse=w.lse, out=out, lse=lse if w.lse else None)
        if ev is not None:
            ev[0][1].record(stream)

    return step, 1, out.element_size(), lambda: accuracy_rows(q, k, v, out, w.causal, None)


def run_timed(args, w, step, S, out_esize, dev, clocks=None, accuracy=None):
    """Warm-up, then exactly args.steps timed steps; prints the JSON line.  step(ev, mev) records
    HIP events around each of its S attention launches (ev[s]) and around the merge (mev).
    accuracy(): output accuracy of the last step on sampled rows.  With --scrub-mib N a buffer of N
    MiB is overwritten before every step (outside that step's events), so each step starts with the
    L2 and the 256 MB MALL holding none of its inputs; the time per step then comes from HIP events
    around each step alone."""
    import torch

    import quantized_attention_quantize_amd as sage

    from quantized_attention_quantize_amd import api as _api

    stream = torch.cuda.current_stream(dev)
    scrub = torch.empty(args.scrub_mib << 20, dtype=torch.uint8, device=dev) if args.scrub_mib > 0 else None

    def pair():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # Everything the timed region needs is made before the first warm-up step, so that from then on
    # the GPU never waits on the host: an idle gap of a few tens of ms before the timed steps makes
    # the chip's power management throttle the next launches (one measured n8k trace: 2.16 ms
    # after a 20 ms gap, settling to 1.55 ms over about 50 ms of load).
    side = torch.cuda.Stream(device=dev)
    clk_buf = torch.zeros(4 * 8, dtype=torch.int64, device=dev)
    evs = [[pair() for _ in range(S)] for _ in range(args.steps)]
    mevs = [pair() for _ in range(args.steps)] if S > 1 else [None] * args.steps
    sevs = [pair() for _ in range(args.steps)] if scrub is not None else None
    g0, g1 = pair()
    wevs = [pair() for _ in range(max(args.warmup, 1))]
    # the clock probe's first launch loads its code (several ms with the GPU idle): done here, once
    try:
        _api.sclk_probe(dev, nblocks=8, iters=1, load=False, stream=side, out=clk_buf)
    except Exception:
        pass
    torch.cuda.synchronize()
    # Warm-up: the W steps back to back, then untimed steps until the loop has kept the GPU busy for
    # SETTLE_S seconds (a synchronization every 8 steps leaves gaps of one launch latency only), so
    # the timed steps start at the clock the chip holds under sustained load.
    tw = time.perf_counter()
    for i in range(args.warmup):
        wevs[i][0].record(stream)
        step()
        wevs[i][1].record(stream)
    settle = 0
    torch.cuda.synchronize()
    while time.perf_counter() - tw < SETTLE_S:
        step()
        settle += 1
        if settle % 8 == 0:
            torch.cuda.synchronize()
    settle_s = time.perf_counter() - tw
    # the fastest warm-up step, for sizing the clock probe below
    warm_ms = min(a.elapsed_time(b) for a, b in wevs[:args.warmup]) if args.warmup > 0 else 1.0
    # the shader clock during the timed steps: idle waves on a second stream read the clock counters
    # over about half of the expected timed window (s_sleep trips of 8128 clocks, <= 3.4 us each)
    clk_iters = max(1, min(int(0.5 * warm_ms * args.steps / 3.4e-3), 1 << 24))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tw0 = time.time()
    g0.record(stream)
    try:
        _api.sclk_probe(dev, nblocks=8, iters=clk_iters, load=False, stream=side, out=clk_buf)
    except Exception:
        clk_buf = None
    for i in range(args.steps):
        if scrub is not None:
            scrub.fill_(i & 255)
            sevs[i][0].record(stream)
        step(evs[i], mevs[i])
        if scrub is not None:
            sevs[i][1].record(stream)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sclk = clocks(tw0, time.time()) if clocks is not None else None
    try:
        probe = _api.sclk_result(clk_buf) if clk_buf is not None else {"error": "probe not launched"}
        probe["source"] = ("sage_sclk_probe (idle form) on a second stream during the timed steps: s_memtime "
                           "against the 100 MHz s_memrealtime over about half of the timed window")
    except Exception as e:  # the measurement aid must not stop the benchmark
        probe = {"error": str(e)}

    ms_step = wall * 1e3 / args.steps
    gpu_ms_step = g0.elapsed_time(g1) / args.steps
    if scrub is not None:  # the steps alone, each after the scrub
        ms_step = sum(a.elapsed_time(b) for a, b in sevs) / args.steps
    attn_ms = sorted(a.elapsed_time(b) for e in evs for a, b in e)  # one entry per attention launch
    attn_avg = sum(attn_ms) / len(attn_ms)
    ops = w.ops
    value = ops / (ms_step * 1e-3) / 1e12
    # the roofline counts the products the kernel has to do: the keys < N/2 masks hide half the keys
    # (the kernel skips their tiles), which the nominal count of the headline metric does not discount
    visible = 0.5 if w.mask in ("half_keys", "half_keys_f32") else 1.0
    achieved = ops * visible / S / (attn_avg * 1e-3) / 1e12  # one launch covers 1/S of the keys
    traffic = traffic_from_profile(w.name, "k_fp4_attn" if w.method == "fp4" else "k_attn_fwd")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"untimed_steps": settle, "seconds": round(settle_s, 3),
                   "rule": f"after the W warm-up steps, untimed steps until the GPU has been busy {SETTLE_S} s"},
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4+f8" if w.method == "fp4" else ("i8+f8" if w.pv == "fp8" else "i8+f16"),
        "data": "synthetic",
        "config": {"workload": w.name, "desc": w.note, "B": w.B, "H": w.H, "Hkv": w.Hkv or w.H, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d,
                   "causal": w.causal, "mask": w.mask, "method": w.method,
                   "pv": "e2m1 V x e4m3 P" if w.method == "fp4" else w.pv, "return_lse": w.lse, "io_dtype": w.dtype,
                   "smooth_v": w.smooth_v, "per_block_mean": w.per_block_mean,
                   "ops_per_step": ops, "pct_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2),
                   "gpu_ms_per_step": round(gpu_ms_step, 4),
                   **({"seqlens": list(w.seqlens)} if w.seqlens else {})},
        "roofline": {"kernel": "k_fp4_attn" if w.method == "fp4" else "k_attn_fwd", "bound": "mfma",
                     "achieved": round(achieved, 2),
                     "peak": round(mfma_peak(w.pv, w.method), 1), "unit": "TOPS",
                     "frac": round(achieved / mfma_peak(w.pv, w.method), 4),
                     "peak_basis": ("dense MFMA: FP4 10100 TOPS for QK^T (e2m1 x e2m1), FP8 5000 TFLOP/s for PV "
                                    "(e2m1 V x e4m3 P runs at the FP8 rate), each half of the counted ops"
                                    if w.method == "fp4" else
                                    "dense MFMA: INT8 5000 TOPS for QK^T, " +
                                    ("FP16 2500 TFLOP/s" if w.pv == "fp16" else "FP8 5000 TFLOP/s") +
                                    " for PV, each half of the counted ops"),
                     "ops_per_launch": ops * visible / S,
                     "traffic": traffic, "avg_ms": round(attn_avg, 4), "median_ms": round(attn_ms[len(attn_ms) // 2], 4),
                     "min_ms": round(attn_ms[0], 4),
                     "timed": ("HIP events around sage_fp4_attn_fwd (k_fp4_attn)" if w.method == "fp4" else
                               "HIP events around sage_attn_fwd_prepared: the mask-tile classification (k_mask_tiles, "
                               "k_mask_walk) and k_attn_fwd" if w.mask else
                               "HIP events around sage_attn_fwd_prepared (k_attn_fwd alone)")},
        "sclk": probe,
        "sclk_sysfs": sclk,
        "accuracy": accuracy() if accuracy is not None else None,
    }
    if scrub is not None:
        line["config"]["cache_scrub_mib"] = args.scrub_mib
        line["config"]["timing"] = "HIP events around each step, a cache scrub before each"
        line["data"] = "synthetic, caches scrubbed before every step"

    if probe.get("median_mhz"):  # the datasheet peaks hold at the 2400 MHz peak engine clock
        f = probe["median_mhz"] / 2400.0
        line["roofline"]["at_measured_sclk"] = {
            "sclk_mhz": probe["median_mhz"], "peak": round(line["roofline"]["peak"] * f, 1),
            "frac": round(line["roofline"]["achieved"] / (line["roofline"]["peak"] * f), 4),
            "basis": "the same MFMA peak scaled by the measured shader clock / 2400 MHz"}
    vc = valu_ceiling(w.name, ops * visible / S, "k_fp4_attn" if w.method == "fp4" else "k_attn_fwd")
    if vc is not None:
        vc["achieved"] = line["roofline"]["achieved"]
        vc["frac"] = round(vc["achieved"] / vc["peak"], 4)
    line["roofline"]["valu"] = vc
    if S > 1:
        merge_ms = sorted(a.elapsed_time(b) for a, b in mevs)
        merge_avg = sum(merge_ms) / len(merge_ms)
        R = w.B * w.H * w.Nq
        mbytes = S * R * w.d * 4 + S * R * 4 + R * w.d * out_esize + (R * 4 if w.lse else 0)
        line["merge_roofline"] = {"kernel": "k_merge_lse", "bound": "hbm", "achieved": round(mbytes / (merge_avg * 1e-3) / 1e9, 1),
                                  "peak": 8000.0, "unit": "GB/s",
                                  "frac": round(mbytes / (merge_avg * 1e-3) / 1e9 / 8000.0, 4),
                                  "bytes_per_launch": mbytes, "avg_ms": round(merge_avg, 4)}
    if not args.no_cpu_baseline:
        # the oracle run with the kernels' online schedule: 64-key tiles, a reference maximum lazy by
        # 8 log2 units for FP16 P and exact for e4m3 P, the denominator over the fp32 probabilities
        tau = 0.0 if (w.method == "fp4" or w.pv == "fp8") else 8.0
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_work, tau, False)
    print(json.dumps(line), flush=True)




def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="n8k")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (5 launches): a kernel of "
                         "known traffic for calibrating HBM byte counters")
    ap.add_argument("--cpu-work", type=float, default=2.7e8,
                    help="query-row x key pairs in the CPU-baseline sample (oracle on the host)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scrub-mib", type=int, default=0,
                    help="overwrite a buffer of this many MiB before every timed step (cold L2 and MALL); the "
                         "time per step is then taken from HIP events around each step")
    ap.add_argument("--sample-clocks", nargs=2, metavar=("OUT", "STOP"), help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.sample_clocks:
        return sample_clocks(*args.sample_clocks)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).  Heads are independent, so N GPUs would each run B*H/N heads of the same "
              f"kernel with no communication.", file=sys.stderr)
        sys.exit(2)

    clocks = start_clock_sampler()  # a child process, started before anything touches the GPU

    import torch

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        clocks(0.0, 0.0)  # stops the sampler
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 5}), flush=True)
        return

    import quantized_attention_quantize_amd as sage
    from quantized_attention_quantize_amd import api
    from quantized_attention_quantize_amd.synthetic import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sage.load_library()
    if w.seqlens or w.method == "fp4":
        step, S, esize, acc = (varlen_setup if w.seqlens else fp4_setup)(w, dev)
        return run_timed(args, w, step, S, esize, dev, clocks, acc)
    inp = workload_inputs(w, seed=0)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    mask = None if inp.mask is None else inp.mask.to(dev)
    del inp

    # every buffer allocated once, outside the timed region
    Hkv = w.Hkv or w.H
    S = w.kv_splits
    bounds = [w.Nk * s // S for s in range(S + 1)]
    if S > 1:  # key slices, resident before timing
        kv = [(k[:, :, lo:hi].contiguous(), v[:, :, lo:hi].contiguous()) for lo, hi in zip(bounds[:-1], bounds[1:])]
    else:
        kv = [(k, v)]
    del k, v
    qks, qwss, vts, vwss, vms = [], [], [], [], []
    for ks, _ in kv:
        nk = ks.shape[2]
        qks.append(api.alloc_quantized(w.B, w.H, w.Nq, nk, w.d, dev, Hkv=Hkv, dtype=q.dtype,
                                       per_block_mean=w.per_block_mean))
        qwss.append(api.quantize_workspace(w.B, Hkv, nk, w.d, dev))
        vts.append(api.alloc_prepared_v(w.B, Hkv, nk, w.d, w.pv, dev))
        vwss.append(api.prepare_v_workspace(w.B, Hkv, nk, w.d, w.pv, dev))
        vms.append(torch.empty(w.B, Hkv, w.d, dtype=torch.float32, device=dev) if w.smooth_v else None)
    mws = api.mask_workspace(w.B, w.Nq, w.Nk, 1 if mask is not None else 0, dev)
    out = torch.empty(w.B, w.H, w.Nq, w.d, dtype=q.dtype, device=dev)
    lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device=dev)
    if S > 1:
        if mask is not None or w.causal:
            raise SystemExit("key-sliced workloads take neither a mask nor causality")
        o_parts = torch.empty(S, w.B, w.H, w.Nq, w.d, dtype=torch.float32, device=dev)
        l_parts = torch.empty(S, w.B, w.H, w.Nq, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None, mev=None):
        for s, (ks, vs_) in enumerate(kv):
            api.quantize_qk(q, ks, out=qks[s], workspace=qwss[s], per_block_mean=w.per_block_mean)
            api.prepare_v(vs_, w.pv, out=vts[s], workspace=vwss[s], v_mean=vms[s])
            if ev is not None:
                ev[s][0].record(stream)
            api.attn_fwd_prepared(qks[s], vts[s][0], vts[s][1], pv_dtype=w.pv, is_causal=w.causal, attn_mask=mask,
                                  return_lse=w.lse or S > 1, out=out if S == 1 else o_parts[s],
                                  lse=lse if S == 1 else l_parts[s], workspace=mws, v_mean=vms[s])
            if ev is not None:
                ev[s][1].record(stream)
        if S > 1:
            if mev is not None:
                mev[0].record(stream)
            api.merge_lse(o_parts, l_parts, out=out, lse=lse if w.lse else None, return_lse=w.lse)
            if mev is not None:
                mev[1].record(stream)

    def accuracy():
        return accuracy_rows(q, kv[0][0] if S == 1 else torch.cat([a for a, _ in kv], 2),
                             kv[0][1] if S == 1 else torch.cat([b for _, b in kv], 2), out, w.causal, mask)

    return run_timed(args, w, step, S, out.element_size(), dev, clocks, accuracy)


if __name__ == "__main__":
    main()
