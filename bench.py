#!/usr/bin/env python
"""Throughput of the quantized attention forward on one MI355X.

One step = the whole hot path on one batch of seeded synthetic input already resident in HBM:
sage_quantize_qk (K mean, INT8 Q/K, scales, LSE shift) -> sage_prepare_v (fp16 or e4m3 V) ->
sage_attn_fwd_prepared (mask classification if any, attention with LSE).

    python bench.py [--steps K] [--warmup W] [--workload n8k]

Prints one JSON line.  ``value`` is attention TOPS = 4*B*H*Nq*Nk*d / (time per step), halved for
causal, over the whole step.  ``roofline`` reports the attention kernel alone: its algorithmic
ops per launch over its average duration, measured with HIP events recorded on the stream the
kernel runs on, against the dense INT8 MFMA peak.  ``cpu_baseline`` times the CPU oracle (the
plain reference implementation used by the tests) on a bounded sample of the same workload.
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
INT8_PEAK_TOPS = 5000.0  # MI355X dense INT8 MFMA (datasheet, no sparsity)
KERNEL_SOURCES = ["quantized_attention_quantize_amd/csrc/sage_attn.hip",
                  "quantized_attention_quantize_amd/csrc/sage_device.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, rows_target: int):
    """The oracle (never tuned) on one head of the workload: K mean, quantization and V preparation
    of that head, then the quantized emulation for `rows_target` query rows of it."""
    import numpy as np

    import oracle
    from quantized_attention_quantize_amd.synthetic import make_inputs

    oracle.build(force=False)
    inp = make_inputs(1, 1, w.Nq, w.Nk, w.d, w.sigma, seed=0, mask=w.mask)
    Qb, Kb, Vb = inp.bits(inp.q), inp.bits(inp.k), inp.bits(inp.v)
    rows = np.linspace(0, w.Nq - 1, min(rows_target, w.Nq)).astype(np.int64)
    t0 = time.perf_counter()
    qk = oracle.quant_qk(Qb, Kb)
    vh, vs = oracle.prep_v(Vb, w.pv)
    oracle.attn_qe(qk, vh, vs, w.pv, w.Nq, w.Nk, causal=w.causal, mask=inp.mask_u8, BN=64, rows=rows)
    dt = time.perf_counter() - t0
    if w.causal:
        ops = float(sum(4.0 * (int(i) + 1) * w.d for i in rows))
    else:  # the mask workload counts formula ops too, as the GPU metric does
        ops = 4.0 * rows.size * w.Nk * w.d
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"1 head (B=1,H=1) of {w.name}: K mean + INT8 quantization + V prep of the head, quantized "
                      f"emulation of {rows.size} evenly spaced query rows x {w.Nk} keys; {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="n8k")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="query rows in the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).  Heads are independent, so N GPUs would each run B*H/N heads of the same "
              f"kernel with no communication.", file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_attention_quantize_amd as sage
    from quantized_attention_quantize_amd import api
    from quantized_attention_quantize_amd.synthetic import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sage.load_library()
    inp = workload_inputs(w, seed=0)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    mask = None if inp.mask is None else inp.mask.to(dev)
    del inp

    # every buffer allocated once, outside the timed region
    qk = api.alloc_quantized(w.B, w.H, w.Nq, w.Nk, w.d, dev)
    qws = api.quantize_workspace(w.B, w.H, w.Nk, w.d, dev)
    vt, vs = api.alloc_prepared_v(w.B, w.H, w.Nk, w.d, w.pv, dev)
    vws = api.prepare_v_workspace(w.B, w.H, w.Nk, w.d, w.pv, dev)
    mws = api.mask_workspace(w.B, w.Nq, w.Nk, 1 if mask is not None else 0, dev)
    out = torch.empty(w.B, w.H, w.Nq, w.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.H, w.Nq, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        api.quantize_qk(q, k, out=qk, workspace=qws)
        api.prepare_v(v, w.pv, out=(vt, vs), workspace=vws)
        if ev is not None:
            ev[0].record(stream)
        api.attn_fwd_prepared(qk, vt, vs, pv_dtype=w.pv, is_causal=w.causal, attn_mask=mask, return_lse=w.lse,
                              out=out, lse=lse, workspace=mws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record(stream)
    for i in range(args.steps):
        step(evs[i])
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = wall * 1e3 / args.steps
    gpu_ms_step = g0.elapsed_time(g1) / args.steps
    attn_ms = sorted(a.elapsed_time(b) for a, b in evs)
    attn_avg = sum(attn_ms) / len(attn_ms)
    ops = w.ops
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (attn_avg * 1e-3) / 1e12
    traffic = traffic_from_profile(w.name)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8+f8" if w.pv == "fp8" else "i8+f16",
        "data": "synthetic",
        "config": {"workload": w.name, "desc": w.note, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "mask": w.mask, "pv": w.pv, "return_lse": w.lse,
                   "ops_per_step": ops, "pct_int8_peak": round(100 * value / INT8_PEAK_TOPS, 2),
                   "gpu_ms_per_step": round(gpu_ms_step, 4)},
        "roofline": {"kernel": "k_attn_fwd", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                     "traffic": traffic, "avg_ms": round(attn_avg, 4), "median_ms": round(attn_ms[len(attn_ms) // 2], 4),
                     "min_ms": round(attn_ms[0], 4)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
