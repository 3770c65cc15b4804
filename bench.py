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
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X published dense bf16 MFMA peak
PEAK_F32_TFLOPS = 157.3      # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0        # MI355X published HBM3E bandwidth
# the attention kernel and every header it is compiled from
KERNEL_SRCS = [os.path.join(ROOT, "context_ring_attention_zigzag_amd", "csrc", f)
               for f in ("attn_bf16.hip", "tile_class.h", "mfma_util.h", "common.h")]
KERNEL_NAME = "attn_bf16_kernel"


def allowed_pairs(w, q_pos, k_pos_all) -> int:
    """Allowed (query, key) pairs of one (b, h), counted from the position arrays."""
    import numpy as np
    q = q_pos[q_pos >= 0]
    k = np.sort(k_pos_all[k_pos_all >= 0])
    if not w.causal:
        return int(len(q)) * int(len(k))
    return int(np.searchsorted(k, q, side="right").sum())


def kernel_hash() -> str:
    """sha256 prefix over the attention kernel's sources, in a fixed order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def field_from_profile(workload: str, kind: str, field: str):
    """A machine-readable field of a committed counter summary, if the summary matches the current kernel."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAME}_{workload}_{kind}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_val = re.search(field + r":\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash():
        return None
    return float(m_val.group(1))


def traffic_from_profile(workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) of the current kernel, or None."""
    return field_from_profile(workload, "traffic", "hbm_bytes_per_launch")


def mfma_busy_from_profile(workload: str):
    """Fraction of the kernel's cycles in which the matrix cores are busy (SQ_VALU_MFMA_BUSY_CYCLES per
    SIMD over GRBM_GUI_ACTIVE per XCD) of the current kernel, or None."""
    return field_from_profile(workload, "counters", "mfma_busy_frac")


def cpu_baseline(w, rank: int, budget_s: float):
    """Time the fp64 oracle on local rows of the workload for about ``budget_s`` seconds.

    Walks (b, h) slices in order and, inside each, the rank's local rows in a seeded order, 64 rows per oracle
    call, until the budget is spent. The rate is allowed-pair flops (4*D per pair) per second of oracle time.
    """
    import numpy as np
    import oracle
    from seeded_inputs import gen_slice
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    lay = {"zigzag": oracle.ZIGZAG, "contiguous": oracle.CONTIGUOUS, "striped": oracle.STRIPED}[w.layout]
    tok, pos = oracle.layout(w.S, w.cp, lay)
    lq = len(tok) // w.cp
    local_pos = pos[rank * lq:(rank + 1) * lq]
    order = np.random.default_rng(0).permutation(lq)
    rows_done, slices, flops, t_used = 0, 0, 0.0, 0.0
    chunk = 64
    for bh in range(w.B * w.H):
        if t_used >= budget_s:
            break
        b, h = divmod(bh, w.H)
        q, k, v = (gen_slice(w, t, b, h)[None, None].astype(np.float64) for t in "qkv")
        slices += 1
        for r0 in range(0, lq, chunk):
            if t_used >= budget_s:
                break
            rows = np.sort(order[r0:r0 + chunk])
            t0 = time.perf_counter()
            oracle.rank_reference(q, k, v, w.S, w.cp, lay, rank, w.causal, rows=rows)
            t_used += time.perf_counter() - t0
            p = local_pos[rows]
            n_keys = np.where(p >= 0, (p + 1) if w.causal else w.S, 0)
            flops += 4.0 * w.D * float(n_keys.sum())
            rows_done += len(rows)
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows_done} local rows of rank {rank} over {slices} (b, h) slice(s) "
                      f"of {w.B * w.H}, fp64 numpy, {t_used:.1f} s of oracle time"}


def measure_state_kernels(cpr, torch, B: int, H: int, Lq: int, D: int, out_dtype, stream, reps: int = 10,
                          q_local=None, q_pos=None):
    """HBM throughput of the state-init, finalize, merge and rotary-embedding kernels at the workload's
    local shape.

    Algorithmic bytes per row: state init writes O (4D) + m, l (8); finalize reads O (4D) + m, l (8) and
    writes O (D*esize) + LSE (4); merge reads two states (8D + 16) and writes one (4D + 8); the rotary
    embedding of the rank's queries
    by their global positions reads and writes one row (2*D*esize) plus its position (4 bytes per row of
    one (b, h)).
    """
    rows = B * H * Lq
    g = torch.Generator(device="cuda").manual_seed(0)
    o = torch.randn((B, H, Lq, D), device="cuda", generator=g)
    m = torch.randn((B, H, Lq), device="cuda", generator=g)
    l = torch.rand((B, H, Lq), device="cuda", generator=g) + 1.0
    o2, m2, l2 = torch.randn_like(o), torch.randn_like(m), torch.rand_like(l) + 1.0
    out = torch.empty((B, H, Lq, D), dtype=out_dtype, device="cuda")
    lse = torch.empty((B, H, Lq), device="cuda")
    esize = out.element_size()
    res = {}
    cases = [("finalize_kernel", lambda: cpr.cp_ring_attn_finalize(o, m, l, out, lse, stream),
              rows * (4 * D + 8 + D * esize + 4)),
             ("merge_kernel", lambda: cpr.cp_ring_attn_merge(o, m, l, o2, m2, l2, stream),
              rows * (8 * D + 16 + 4 * D + 8))]
    o3, m3, l3 = torch.empty_like(o), torch.empty_like(m), torch.empty_like(l)
    cases.append(("state_init_kernel", lambda: cpr.cp_ring_attn_init(o3, m3, l3, stream), rows * (4 * D + 8)))
    if q_local is not None:
        cases.append(("rope_kernel", lambda: cpr.cp_rope_apply(q_local, q_pos, out=out, stream=stream),
                      rows * 2 * D * esize + Lq * 4))
    for name, fn, nbytes in cases:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": nbytes, "kernel_ms": round(ms, 4)}
    return res


def layout_balance(args, cpr, di, torch, w, gen_slice, lay_codes):
    """Per-rank time of the fused ring pass for each layout at one causal workload shape.

    The causal split is what the layouts are about: a contiguous split leaves
    the later ranks with more allowed pairs ("Context Parallelism v.s. Sequence
    Parallelism (Megatron-LM)", "Implementation quirk: symmetric chunk
    assignment"); zigzag and striped assignment even them out ("Sequence
    Parallelism and Ring Attention", "The future of sequence parallelism and
    ring attention"). Every rank is emulated on this one GPU, one after another.
    """
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    nat = {t: di.upload(lambda b, h, t=t: gen_slice(w, t, b, h), w.B, w.H, w.S, w.D, tdt) for t in "qkv"}
    stream = torch.cuda.current_stream()
    out = {}
    for name in ("contiguous", "zigzag", "striped"):
        lay = lay_codes[name]
        tok, pos = di.layout_arrays(w.S, w.cp, lay)
        per_rank = []
        for rank in range(w.cp):
            ri = di.prepare_rank(nat["q"], nat["k"], nat["v"], w.S, w.cp, lay, rank, tok, pos)
            o = torch.empty_like(ri.q_local)
            lse = torch.empty(ri.q_local.shape[:3], dtype=torch.float32, device="cuda")
            pairs = allowed_pairs(w, ri.q_pos.cpu().numpy(), ri.ring_pos.cpu().numpy())

            def run():
                cpr.cp_ring_attn_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, True, 0.0,
                                     o, lse, None, cpr.RUN_FUSED, stream)
            for _ in range(args.warmup):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(args.steps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            flop = 4.0 * w.B * w.H * w.D * pairs
            per_rank.append({"rank": rank, "ms": round(ms, 4), "pairs_per_bh": pairs,
                             "tflops": round(flop / (ms * 1e-3) / 1e12, 1)})
            del ri, o, lse
        slowest = max(p["ms"] for p in per_rank)
        out[name] = {"per_rank": per_rank, "slowest_ms": slowest,
                     "slowest_over_mean": round(slowest / (sum(p["ms"] for p in per_rank) / len(per_rank)), 3)}
    print(json.dumps({"layout_balance": out,
                      "config": {"B": w.B, "H": w.H, "D": w.D, "seq_len": w.S, "cp_size": w.cp, "causal": True,
                                 "dtype": w.dtype, "steps": args.steps, "warmup": args.warmup},
                      "data": "synthetic: seeded N(0,1) draws per (tensor, b, h) slice"}), flush=True)


def bench_backward(args, cpr, di, torch, w, gen_slice, lay_codes):
    """Time one rank's backward ring pass: preprocessing, dQ over every block, the rank's share of every
    block's dK and dV. Inputs: the same seeded Q, K, V as the forward measurement plus a seeded dO; O and
    LSE from the library's own forward pass (timing only, nothing is checked here)."""
    rank = w.ranks[0] if args.rank is None else args.rank
    lay = lay_codes[w.layout]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    nat = {t: di.upload(lambda b, h, t=t: gen_slice(w, t, b, h), w.B, w.H, w.S, w.D, tdt) for t in ("q", "k", "v", "do")}
    tok, pos = di.layout_arrays(w.S, w.cp, lay)
    ri = di.prepare_rank(nat["q"], nat["k"], nat["v"], w.S, w.cp, lay, rank, tok, pos)
    do_local = di.gather(nat["do"], w.S, tok[rank * ri.lq:(rank + 1) * ri.lq])
    del nat
    o = torch.empty_like(ri.q_local)
    lse = torch.empty(ri.q_local.shape[:3], dtype=torch.float32, device="cuda")
    cpr.cp_ring_attn_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, w.causal, 0.0, o, lse)
    dq = torch.empty(ri.q_local.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(ri.k_ring.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(ri.v_ring.shape, dtype=torch.float32, device="cuda")
    # sized for the split of a grid too small for the GPU (equals the base size for large grids)
    ws_bytes = cpr.cp_ring_attn_bwd_workspace_size_ex(w.B, w.H, w.H, w.D, ri.lq, w.cp * ri.lq)
    split = ws_bytes > cpr.cp_ring_attn_bwd_workspace_size(w.B, w.H, ri.lq)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    pairs = allowed_pairs(w, ri.q_pos.cpu().numpy(), ri.ring_pos.cpu().numpy())
    # FlashAttention convention: the backward is 2.5 forward passes (S recomputed, dP, dV, dQ, dK)
    flop = 10.0 * w.B * w.H * w.D * pairs
    stream = torch.cuda.current_stream()

    def step():
        cpr.cp_ring_attn_bwd_run(ri.q_local, ri.q_pos, ri.k_ring, ri.v_ring, ri.ring_pos, w.cp, rank, o, do_local,
                                 lse, w.causal, 0.0, dq, dk, dv, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    value = flop / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    line = {
        "metric": "per-rank ring-attention backward TFLOP/s (10*D flop per allowed pair); % of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic: seeded N(0,1) draws per (tensor, b, h) slice, dO included",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "D": w.D, "seq_len": w.S,
                   "cp_size": w.cp, "layout": w.layout, "rank": rank, "causal": w.causal, "local_queries": ri.lq,
                   "allowed_pairs_per_bh": pairs, "small_grid_split": bool(split)},
        "roofline": {"bound": "mfma" if w.dtype == "bf16" else "alu", "achieved": round(value, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(value / peak, 4), "traffic": None,
                     "kernel": "bwd_prep + bwd_dq_kernel + bwd_dkv_kernel" + (" (split) + bwd_reduce_kernel"
                                                                             if split else "") + " (one call)",
                     "kernel_ms": round(ms, 4),
                     "flop_per_launch": flop},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1, help="GPUs of the run; only 1 is supported")
    ap.add_argument("--steps", type=int, default=20, help="timed passes")
    ap.add_argument("--warmup", type=int, default=3, help="untimed passes before them")
    ap.add_argument("--workload", default="longdoc_noncausal",
                    help="longdoc_noncausal (default), seq32k_cp4, million_cp8, example_4k, ...")
    ap.add_argument("--rank", type=int, default=None, help="the rank to emulate (default: the workload's)")
    ap.add_argument("--stepwise", action="store_true",
                    help="time the stepwise run (one step launch per ring block, the first from the empty state, "
                         "the last writing the output) instead of the fused one")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of CPU oracle work (0 = skip)")
    ap.add_argument("--layout-balance", action="store_true",
                    help="time every rank of the 32k-token causal sequence under the contiguous, zigzag and striped "
                         "layouts (one JSON line) instead of the default measurement")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward"), default="forward",
                    help="backward: time the rank's backward ring pass (cp_ring_attn_bwd_run) on the same workload "
                         "instead of the forward pass")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1).",
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

    LAY_CODES = {"zigzag": cpr.ZIGZAG, "contiguous": cpr.CONTIGUOUS, "striped": cpr.STRIPED}
    if args.layout_balance:
        layout_balance(args, cpr, di, torch, WORKLOADS["seq32k_cp4"], gen_slice, LAY_CODES)
        return

    w = WORKLOADS[args.workload]
    if args.which == "backward":
        bench_backward(args, cpr, di, torch, w, gen_slice, LAY_CODES)
        return
    rank = w.ranks[0] if args.rank is None else args.rank
    lay = LAY_CODES[w.layout]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    t_prep = time.perf_counter()
    nat = {t: di.upload(lambda b, h, t=t: gen_slice(w, t, b, h), w.B, w.H, w.S, w.D, tdt) for t in "qkv"}
    tok, pos = di.layout_arrays(w.S, w.cp, lay)
    ri = di.prepare_rank(nat["q"], nat["k"], nat["v"], w.S, w.cp, lay, rank, tok, pos)
    del nat
    o = torch.empty_like(ri.q_local)
    lse = torch.empty(ri.q_local.shape[:3], dtype=torch.float32, device="cuda")
    flags = cpr.RUN_STEPWISE if args.stepwise else cpr.RUN_FUSED
    # the workspace holds the stepwise state, or the partial states of a fused run whose grid is too small
    # for the GPU and is split over the keys (allocated before the timed region)
    ws_bytes = cpr.cp_ring_attn_workspace_size(w.B, w.H, ri.lq, w.D)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    kv_split = 1 if (args.stepwise or w.dtype != "bf16") else ws_bytes // (w.B * w.H * ri.lq * (w.D + 2) * 4)
    torch.cuda.synchronize()
    t_prep = time.perf_counter() - t_prep

    pos_h = ri.ring_pos.cpu().numpy()
    pairs = allowed_pairs(w, ri.q_pos.cpu().numpy(), pos_h)
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
                "kernel": (KERNEL_NAME if kv_split == 1 else f"{KERNEL_NAME} (keys split {kv_split} ways) + "
                           "merge_finalize_kernel") if w.dtype == "bf16" else "attn_f32_kernel",
                "kernel_ms": round(kernel_ms, 4), "flop_per_launch": flop,
                "mfma_busy_frac": mfma_busy_from_profile(w.name) if kv_split == 1 else None,
                "kernel_source_sha256_16": kernel_hash()}

    state_kernels = measure_state_kernels(cpr, torch, w.B, w.H, ri.lq, w.D, tdt, stream, q_local=ri.q_local,
                                          q_pos=ri.q_pos)

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
                   "kv_split": int(kv_split),
                   "input_prep_s": round(t_prep, 1)},
        "roofline": roofline,
        "state_kernels": state_kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
