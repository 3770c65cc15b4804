"""Benchmark: one context-parallel rank's ring-attention pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: the layout build (cp_zigzag_partition) followed by
cp_ring_attn_run (every ring block folded, then the output normalised).
The default workload is the non-causal long-document share (B=2, H=16, D=128,
S=65536 over cp=8 contiguous ranks, rank 0, inputs N(0,1)*0.5 in bf16).

Prints one JSON line with the causal-effective TFLOP/s (4*B*H*D per allowed
(query, key) pair), the roofline of the attention kernel (timed with HIP
events on the stream it runs on) and the fp64 CPU oracle's rate on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X published dense bf16 MFMA peak
PEAK_F32_TFLOPS = 157.3      # MI355X published fp32 vector peak
KERNEL_SRC = os.path.join(ROOT, "context_ring_attention_zigzag_amd", "csrc", "attn_bf16.hip")
KERNEL_NAME = "attn_bf16_kernel"


def allowed_pairs(w, s_pad: int, lq: int, q_pos, k_pos_all) -> int:
    """Allowed (query, key) pairs of one (b, h), counted from the position arrays."""
    import numpy as np
    q = q_pos[q_pos >= 0]
    k = np.sort(k_pos_all[k_pos_all >= 0])
    if not w.causal:
        return int(len(q)) * int(len(k))
    return int(np.searchsorted(k, q, side="right").sum())


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernel."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAME}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, rank: int, budget_s: float):
    """Time the fp64 oracle on sampled local rows of one (b, h) slice for about ``budget_s`` seconds."""
    import numpy as np
    import oracle
    from seeded_inputs import gen_slice
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    lay = oracle.ZIGZAG if w.layout == "zigzag" else oracle.CONTIGUOUS
    q = gen_slice(w, "q", 0, 0)[None, None].astype(np.float64)
    k = gen_slice(w, "k", 0, 0)[None, None].astype(np.float64)
    v = gen_slice(w, "v", 0, 0)[None, None].astype(np.float64)
    tok, pos = oracle.layout(w.S, w.cp, lay)
    lq = len(tok) // w.cp
    local_pos = pos[rank * lq:(rank + 1) * lq]
    rng = np.random.default_rng(0)
    order = rng.permutation(lq)
    done, flops, t_used = 0, 0.0, 0.0
    chunk = 64
    while t_used < budget_s and done < lq:
        rows = np.sort(order[done:done + chunk])
        t0 = time.perf_counter()
        oracle.rank_reference(q, k, v, w.S, w.cp, lay, rank, w.causal, rows=rows)
        t_used += time.perf_counter() - t0
        p = local_pos[rows]
        n_keys = np.where(p >= 0, (p + 1) if w.causal else w.S, 0)
        flops += 4.0 * w.D * float(n_keys.sum())
        done += len(rows)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {lq} local rows of (b=0, h=0), rank {rank}, fp64 numpy, {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="longdoc_noncausal")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--stepwise", action="store_true", help="time the init/step/finalize path instead of the fused one")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import context_ring_attention_zigzag_amd as cpr
    from context_ring_attention_zigzag_amd import device_inputs as di
    from seeded_inputs import WORKLOADS, gen_slice

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cpr.load()

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    w = WORKLOADS[args.workload]
    rank = w.ranks[0] if args.rank is None else args.rank
    lay = cpr.ZIGZAG if w.layout == "zigzag" else cpr.CONTIGUOUS
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    t_prep = time.perf_counter()
    nat = {t: di.upload(lambda b, h, t=t: gen_slice(w, t, b, h), w.B, w.H, w.S, w.D, tdt) for t in "qkv"}
    tok, pos = di.layout_arrays(w.S, w.cp, lay)
    ri = di.prepare_rank(nat["q"], nat["k"], nat["v"], w.S, w.cp, lay, rank, tok, pos)
    del nat
    o = torch.empty_like(ri.q_local)
    lse = torch.empty(ri.q_local.shape[:3], dtype=torch.float32, device="cuda")
    ws = None
    flags = cpr.RUN_FUSED
    if args.stepwise:
        flags = cpr.RUN_STEPWISE
        ws = torch.empty(cpr.cp_ring_attn_workspace_size(w.B, w.H, ri.lq, w.D), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t_prep = time.perf_counter() - t_prep

    pos_h = ri.ring_pos.cpu().numpy()
    pairs = allowed_pairs(w, ri.s_pad, ri.lq, ri.q_pos.cpu().numpy(), pos_h)
    flop = 4.0 * w.B * w.H * w.D * pairs

    stream = torch.cuda.current_stream()

    def step(ev=None):
        cpr.cp_zigzag_partition(w.S, w.cp, lay, tok, pos, stream)
        if ev is not None:
            ev[0].record(stream)
        cpr.cp_ring_attn_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, w.causal, 0.0,
                             o, lse, ws, flags, stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(kev[i])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / args.steps
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    roofline = {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic_from_profile(w.name),
                "kernel": KERNEL_NAME if w.dtype == "bf16" else "attn_f32_kernel",
                "kernel_ms": round(kernel_ms, 4), "flop_per_launch": flop}

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(w, rank, args.cpu_budget)
        cpu["value"] = round(cpu["value"], 6)

    line = {
        "metric": "per-rank ring-attention causal-effective TFLOP/s; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) draws per (tensor, b, h) slice, scaled and rounded to the input dtype",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "seq_len": w.S, "cp_size": w.cp,
                   "layout": w.layout, "rank": rank, "causal": w.causal, "local_queries": ri.lq,
                   "allowed_pairs_per_bh": pairs, "run_mode": "stepwise" if args.stepwise else "fused",
                   "input_prep_s": round(t_prep, 1)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
