#!/usr/bin/env python3
"""Throughput of the sparse + linear attention forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the K/V preparation pass (sla_kv_prepare, which also pools K for the mask),
the block mask (sla_mask_prepared) and the fused sparse + linear + alpha-mix
kernel (sla_fused_fwd) - the same launches as sla_attn_fwd, issued one by one
so that HIP events on the launch stream bracket each stage.  Inputs are
resident in HBM before timing starts.

Cache control.  Q, K and V of the 480p workload (302 MB) nearly fit the
256 MB last-level cache, so the timed steps rotate over --sets copies of the
inputs (default 3): every step reads inputs that the two steps before it did
not touch, and `value` is that cold-input rate.  The same steps on one input
set are reported as `warm`.

Clock.  A GPU that was idle takes tens of milliseconds of load before its
shader clock settles; steps timed in that window run 10-15% slower.  Before
the --warmup steps the bench therefore runs untimed steps for --settle-s
seconds (reported under `settle`).

Prints ONE JSON line.  value = dense-equivalent TFLOP/s = 4 B H N^2 d /
(time per step).  The roofline object covers the fused kernel: algorithmic
FLOPs (4 bq bk d per executed (query block, key block) pair plus 2 bq d^2 per
query block with a linear branch) over its mean launch time, with the matrix
work the kernel actually executes beside it.  The mask roofline covers the
standalone mask call sla_mask (Q and K read once, the CSR written once).  The
dense comparators are this library's dense kernel and torch's
scaled_dot_product_attention (a fused backend, labelled external), both on
the same tensors.  cpu_baseline times the fp64 oracle stage by stage on a
bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dense-equivalent attention TFLOPS + speedup vs dense at 97% sparsity, N=32760"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_I8_TOPS = 5000.0          # MI355X dense int8 matrix peak
FUSED_SRC = os.path.join(ROOT, "block_sparse_linear_sla_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_fused_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="untimed steps for this many seconds before the warm-up (clock settle)")
    ap.add_argument("--sets", type=int, default=3, help="input copies the timed steps rotate over")
    ap.add_argument("--workload", default="video480p-sla2-N32760")
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time spent on the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the 8-bit, backward and SoftTop-k legs")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the leg that replays the step as captured HIP graphs")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def src_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic():
    """Fused-kernel HBM bytes per launch from the committed counter runs, or
    None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha256_16") != src_digest(FUSED_SRC):
        return None
    return t.get("bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, budget_s: float):
    """The fp64 oracle as it stands, stage by stage, on a bounded sample of
    the workload: the whole mask of head (0, 0), then the sparse branch, the
    linear branch (heads whose alpha is 1 skip it, as in the oracle's own
    forward) and the combine of M random query blocks of that head.  M is
    sized from a one-block probe so that three runs fill about 3/4 of the
    budget; the stage times are the median of the three runs with every BLAS
    thread, and a fourth run on max(2, M/8) blocks with one thread gives the
    single-thread rate.  value = dense-equivalent FLOPs of one query block
    (4 bq N d) / (mask time per block + branch time per block)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import sla_oracle as O
    wl = x.wl
    q1, k1, v1 = (t[:1, :1].to("cpu").double().numpy() for t in (x.Q, x.K, x.V))
    wq = None if x.Wq is None else x.Wq.double().numpy()
    wk = None if x.Wk is None else x.Wk.double().numpy()
    a0 = float(x.alpha[0])
    rng = np.random.default_rng(0)
    order = [int(i) for i in rng.permutation(wl.Nq)]
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    threads = int(blas[0]["num_threads"]) if blas else 1
    vendor = (f"{blas[0].get('internal_api')} {blas[0].get('version')} ({blas[0].get('architecture')}, "
              f"{blas[0].get('threading_layer')})") if blas else "unknown"

    def run(n_rows):
        t0 = time.perf_counter()
        rp, ci, _ = O.mask(q1, k1, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, keep_info=False)
        t = {"mask": time.perf_counter() - t0}
        rows = [(0, 0, i) for i in order[:n_rows]]
        t0 = time.perf_counter()
        os_ = O.sparse_branch(q1, k1, v1, wl.bq, wl.bk, rp, ci, rows) if a0 != 0.0 else {}
        t["sparse"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        ol = O.linear_branch(q1, k1, v1, wl.bq, wl.bk, rp, ci, rows) if a0 != 1.0 else {}
        t["linear"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        for r in rows:
            z = np.zeros((O.block_range(r[2], wl.bq, wl.N)[1] - O.block_range(r[2], wl.bq, wl.N)[0], wl.d))
            O.combine(os_.get(r, z), ol.get(r, z), a0)
        t["combine"] = time.perf_counter() - t0
        return t

    probe = run(1)
    per_row = probe["sparse"] + probe["linear"] + probe["combine"]
    M = int(max(2, min(wl.Nq, (0.25 * budget_s - probe["mask"]) / max(per_row, 1e-6))))
    runs = [run(M) for _ in range(3)]
    med = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
    M1 = max(2, M // 8)
    with threadpool_limits(limits=1):
        one = run(M1)
    flops_block = 4.0 * wl.bq * wl.N * wl.d          # dense-equivalent work of one query block

    def rate(t, n):
        per_block = t["mask"] / wl.Nq + (t["sparse"] + t["linear"] + t["combine"]) / n
        return flops_block / per_block / 1e12

    return {"value": rate(med, M), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 numpy oracle on head (0,0) of {wl.name}: the head's whole mask ({wl.Nq} query "
                       f"blocks) + sparse branch, linear branch and combine of {M} random query blocks; "
                       f"median of 3 runs; value = dense-equivalent FLOPs per query block (4*bq*N*d) / "
                       f"(mask time per block + branch time per block)"),
            "stage_s_median": med, "rows": M,
            "one_thread": {"value": rate(one, M1), "rows": M1, "stage_s": one},
            "cpu_model": _cpu_model(), "blas": vendor, "blas_threads": threads,
            "host_cpus": len(os.sched_getaffinity(0))}


def sdpa_leg(q, k, v, steps, ref):
    """torch.nn.functional.scaled_dot_product_attention on the same bf16
    tensors with a fused backend (flash, else memory-efficient); never the
    math fallback.  Returns its mean time and its largest difference from
    this library's dense output `ref`, or the error text."""
    import torch
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    last = None
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                o = F.scaled_dot_product_attention(q, k, v)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(steps):
                    o = F.scaled_dot_product_attention(q, k, v)
                e1.record()
                torch.cuda.synchronize()
            diff = (o.float() - ref.float()).abs().max().item() if ref is not None else None
            return {"ms": e0.elapsed_time(e1) / steps, "backend": name, "max_abs_vs_library_dense": diff}
        except RuntimeError as err:  # backend unavailable for this shape or build
            last = f"{name}: {err}"
    return {"ms": None, "error": (last or "")[:300]}


def timed_steps(step, n, sets, events_per_step=4):
    """n steps, step(i, set, events); HIP events on the launch stream around
    each stage.  Returns (wall ms per step, per-stage mean ms list)."""
    import torch
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(events_per_step)] for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        step(i % sets, events[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n * 1e3
    stages = [sum(e[j].elapsed_time(e[j + 1]) for e in events) / n for j in range(events_per_step - 1)]
    stages.append(sum(e[0].elapsed_time(e[-1]) for e in events) / n)
    return wall, stages


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards over (batch, head) with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_linear_sla_amd as S
    import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    S.lib()
    wl = gen.WORKLOADS[args.workload]
    x = gen.make(wl)
    dev = torch.device("cuda:0")
    nset = max(1, args.sets)
    q, k, v, alpha = (t.to(dev).contiguous() for t in (x.Q, x.K, x.V, x.alpha))
    sets = [(q, k, v)] + [(q.clone(), k.clone(), v.clone()) for _ in range(nset - 1)]
    wq = None if x.Wq is None else x.Wq.to(dev)
    wk = None if x.Wk is None else x.Wk.to(dev)
    prob, sel = S.problem(q, wl.bq, wl.bk), S.select(wl.k_frac, wl.p, wq, wk)
    ws = S.workspace(prob, sel, dev)
    cap = S.sla_mask_capacity(prob)
    rp = torch.empty(wl.B * wl.H * wl.Nq + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(cap, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    def step(si, ev=None):
        qq, kk, vv = sets[si]
        if ev is not None:
            ev[0].record()
        S.sla_kv_prepare(kk, vv, wl.bq, wl.bk, ws, alpha)
        if ev is not None:
            ev[1].record()
        S.sla_mask_prepared(qq, kk, alpha, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, ws=ws, row_ptr=rp, col_idx=ci)
        if ev is not None:
            ev[2].record()
        S.sla_fused_fwd(qq, kk, vv, alpha, wl.bq, wl.bk, rp, ci, ws, out=out)
        if ev is not None:
            ev[3].record()

    # clock settle: untimed steps for settle_s seconds, in bursts of 16
    n_settle, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_s:
        for _ in range(16):
            step(n_settle % nset)
            n_settle += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t0) * 1e3
    for i in range(args.warmup):
        step(i % nset)
    torch.cuda.synchronize()
    ms_step, (st_sum, st_maskp, st_fused, ev_step) = timed_steps(step, args.steps, nset)
    ms_warm, (w_sum, w_maskp, w_fused, w_ev) = timed_steps(step, args.steps, 1)

    # the same step captured once per input set as a HIP graph and replayed
    # in the same rotation: what a caller that replays graphs sees (the
    # library only launches kernels, so a step captures whole)
    graph = None
    if not args.no_graph:
        try:
            graphs = []
            for si in range(nset):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(si)
                graphs.append(g)
            for i in range(10):
                graphs[i % nset].replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for i in range(args.steps):
                graphs[i % nset].replay()
            e1.record()
            torch.cuda.synchronize()
            graph = {"ms_per_step": e0.elapsed_time(e1) / args.steps, "steps": args.steps, "input_sets": nset}
            del graphs
        except RuntimeError as err:  # reported, never fatal: the eager figures stand on their own
            graph = {"error": str(err)[:200]}

    # the standalone mask call (pools Q and K itself), for the mask's HBM
    # roofline: rotating over the input sets (cold) and on one set (warm)
    rp_m, ci_m = torch.empty_like(rp), torch.empty_like(ci)

    def mask_call(si, ev=None):
        if ev is not None:
            ev[0].record()
        S.sla_mask(sets[si][0], sets[si][1], wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, ws=ws, row_ptr=rp_m,
                   col_idx=ci_m)
        if ev is not None:
            ev[1].record()

    for i in range(10):
        mask_call(i % nset)
    _, (st_mask, _) = timed_steps(mask_call, args.steps, nset, events_per_step=2)
    _, (st_mask_warm, _) = timed_steps(mask_call, args.steps, 1, events_per_step=2)
    n_m = int(rp_m[-1])
    if not (torch.equal(rp_m, rp) and torch.equal(ci_m[:n_m], ci[:n_m])):
        raise RuntimeError("sla_mask and sla_mask_prepared disagree")

    # algorithmic work from the mask this step produced
    counts = np.diff(rp.cpu().numpy().astype(np.int64))
    nnz = int(counts.sum())
    a = x.alpha.numpy().astype(np.float64)
    heads = np.repeat(np.tile(np.arange(wl.H), wl.B), wl.Nq)
    s_rows = a[heads] != 0.0
    l_rows = (a[heads] != 1.0) & (counts < wl.Nk)
    pair_flops = 4.0 * wl.bq * wl.bk * wl.d
    fused_flops = pair_flops * counts[s_rows].sum() + 2.0 * wl.bq * wl.d * wl.d * l_rows.sum()
    # matrix work the fused kernel executes: S and P V per listed pair of a
    # row with the sparse branch; G = phi(K)^T V per listed pair and the
    # three-product phi(Q) H_u per row with the linear branch
    exec_flops = (pair_flops * counts[s_rows].sum() + 2.0 * wl.bk * wl.d * wl.d * counts[l_rows].sum()
                  + 3 * 2.0 * wl.bq * wl.d * wl.d * l_rows.sum())
    dense_flops = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.d
    es = 2 if wl.dtype == "bf16" else 4
    mask_bytes = 2.0 * wl.B * wl.H * wl.N * wl.d * es + 4.0 * (len(counts) + 1) + 4.0 * nnz

    def tf(flops, ms):
        return flops / (ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": dense_flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "bq": wl.bq,
                   "bk": wl.bk, "k_frac": wl.k_frac, "p": wl.p, "grid_thw": list(wl.grid),
                   "router": wl.router, "seed": wl.seed, "input_sets": nset},
        "roofline": {"bound": "mfma", "achieved": tf(fused_flops, st_fused),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf(fused_flops, st_fused) / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(), "kernel": f"attn_kernel<d={wl.d},bq={wl.bq},bk={wl.bk},fused>",
                     "flops_per_launch": fused_flops, "ms_per_launch": st_fused,
                     "executed_flops_per_launch": exec_flops,
                     "executed_achieved": tf(exec_flops, st_fused),
                     "executed_frac": tf(exec_flops, st_fused) / PEAK_BF16_TFLOPS},
        "mask_roofline": {"bound": "hbm", "achieved": mask_bytes / (st_mask * 1e-3) / 1e9,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": mask_bytes / (st_mask * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "bytes_per_call": mask_bytes, "ms_per_call": st_mask,
                          "warm_ms_per_call": st_mask_warm,
                          "warm_achieved": mask_bytes / (st_mask_warm * 1e-3) / 1e9},
        "stage_ms": {"kv_prepare": st_sum, "mask_prepared": st_maskp, "fused": st_fused,
                     "events_step": ev_step, "mask_standalone": st_mask},
        "warm": {"ms_per_step": ms_warm, "value": dense_flops / (ms_warm * 1e-3) / 1e12,
                 "stage_ms": {"kv_prepare": w_sum, "mask_prepared": w_maskp, "fused": w_fused,
                              "events_step": w_ev}},
        "settle": {"ms": settle_ms, "steps": n_settle},
        "graph": graph,
        "sparsity": 1.0 - nnz / float(wl.B * wl.H * wl.Nq * wl.Nk), "nnz": nnz,
        "executed_TFLOPS_fused": tf(fused_flops, st_fused),
    }

    if not args.no_dense:
        ref = torch.empty_like(q)
        S.sla_dense_fwd(q, k, v, wl.bq, wl.bk, out=ref)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_steps):
            S.sla_dense_fwd(q, k, v, wl.bq, wl.bk, out=out)
        e1.record()
        torch.cuda.synchronize()
        t_dense = e0.elapsed_time(e1) / args.dense_steps
        res["dense_ms"] = t_dense
        res["dense_TFLOPS"] = dense_flops / (t_dense * 1e-3) / 1e12
        res["speedup_vs_dense"] = t_dense / ms_step
        if wl.dtype == "bf16":
            ext = sdpa_leg(q, k, v, args.dense_steps, ref)
            res["dense_external"] = ext
            if ext.get("ms"):
                res["dense_external_ms"] = ext["ms"]
                res["dense_external_TFLOPS"] = dense_flops / (ext["ms"] * 1e-3) / 1e12
                res["speedup_vs_dense_external"] = ext["ms"] / ms_step
        del ref

    # the sparse branch alone (sla_sparse_fwd) on this step's mask, for the
    # executed-block rate of the attention kernel
    S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci, out=out)
    e1.record()
    torch.cuda.synchronize()
    t_sp = e0.elapsed_time(e1) / args.steps
    res["sparse_fwd_ms"] = t_sp
    res["sparse_fwd_executed_TFLOPS"] = pair_flops * nnz / (t_sp * 1e-3) / 1e12

    # the 8-bit sparse branch on the same mask: quantisation of Q, K, V, then
    # the two-pass int8 kernel; its algorithmic rate (4 bq bk d operations per
    # executed pair) is priced against the int8 matrix peak
    if wl.dtype == "bf16" and not args.no_extras:
        qbuf = S.sla_quantize_i8(q, k, v, wl.bq, wl.bk)
        S.sla_sparse_fwd_i8(qbuf, q, wl.bq, wl.bk, rp, ci, out=out)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(args.steps):
            S.sla_quantize_i8(q, k, v, wl.bq, wl.bk, out=qbuf)
        e[1].record()
        for _ in range(args.steps):
            S.sla_sparse_fwd_i8(qbuf, q, wl.bq, wl.bk, rp, ci, out=out)
        e[2].record()
        torch.cuda.synchronize()
        t_q = e[0].elapsed_time(e[1]) / args.steps
        t_i8 = e[1].elapsed_time(e[2]) / args.steps
        i8_ops = pair_flops * nnz
        res["i8"] = {"quantize_ms": t_q, "sparse_fwd_i8_ms": t_i8,
                     "achieved": i8_ops / (t_i8 * 1e-3) / 1e12, "peak": PEAK_I8_TOPS, "unit": "TOP/s",
                     "frac": i8_ops / (t_i8 * 1e-3) / 1e12 / PEAK_I8_TOPS,
                     "kernel": f"attn_i8_kernel<d={wl.d},bq={wl.bq},bk={wl.bk}>",
                     "vs_bf16_sparse": t_sp / t_i8, "with_quantize_vs_bf16_sparse": t_sp / (t_q + t_i8)}
        # the single-pass 8-bit branch (int8 scores, E4M3 P and V) on the
        # same mask: half its matrix work is int8, half E4M3, both priced at
        # the 5 POP/s (int8) = 5 PFLOP/s (fp8) dense peak
        qb2 = S.sla_quantize_i8f8(q, k, v, wl.bq, wl.bk)
        S.sla_sparse_fwd_i8f8(qb2, q, wl.bq, wl.bk, rp, ci, out=out)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(args.steps):
            S.sla_quantize_i8f8(q, k, v, wl.bq, wl.bk, out=qb2)
        e[1].record()
        for _ in range(args.steps):
            S.sla_sparse_fwd_i8f8(qb2, q, wl.bq, wl.bk, rp, ci, out=out)
        e[2].record()
        torch.cuda.synchronize()
        t_q2 = e[0].elapsed_time(e[1]) / args.steps
        t_f8 = e[1].elapsed_time(e[2]) / args.steps
        res["i8f8"] = {"quantize_ms": t_q2, "sparse_fwd_i8f8_ms": t_f8,
                       "achieved": i8_ops / (t_f8 * 1e-3) / 1e12, "peak": PEAK_I8_TOPS, "unit": "TOP/s",
                       "frac": i8_ops / (t_f8 * 1e-3) / 1e12 / PEAK_I8_TOPS,
                       "kernel": f"attn_i8f8_kernel<d={wl.d},bq={wl.bq},bk={wl.bk}>",
                       "vs_bf16_sparse": t_sp / t_f8, "with_quantize_vs_bf16_sparse": t_sp / (t_q2 + t_f8)}

    # the sparse branch's backward (mask fixed) on this step's mask: the mask
    # transpose, the dQ pass and the dK/dV pass.  Algorithmic work: the five
    # matrix products of a softmax-attention gradient per executed pair
    # (S, dP, dV, dQ, dK: 10 bq bk d), priced against the bf16 matrix peak
    if wl.dtype == "bf16" and not args.no_extras:
        dO = torch.randn_like(q)
        bws = S.bwd_workspace(S.problem(q, wl.bq, wl.bk), dev)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        S.sla_sparse_bwd(q, k, v, dO, wl.bq, wl.bk, rp, ci, ws=bws, out=grads)
        torch.cuda.synchronize()
        S.sla_linear_bwd(q, k, v, dO, wl.bq, wl.bk, rp, ci, ws=bws, out=grads, accumulate=True)
        torch.cuda.synchronize()
        S.sla_attn_bwd(q, k, v, dO, alpha, wl.bq, wl.bk, rp, ci, ws=bws, out=grads)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record()
        for _ in range(args.steps):
            S.sla_sparse_bwd(q, k, v, dO, wl.bq, wl.bk, rp, ci, ws=bws, out=grads)
        e[1].record()
        for _ in range(args.steps):
            S.sla_alpha_grad(dO, out, grads[0], wl.bq, wl.bk, ws=bws)
        e[2].record()
        for _ in range(args.steps):
            S.sla_linear_bwd(q, k, v, dO, wl.bq, wl.bk, rp, ci, ws=bws, out=grads, accumulate=True)
        e[3].record()
        da0 = torch.empty(wl.H, dtype=torch.float32, device=dev)
        for _ in range(args.steps):
            S.sla_attn_bwd(q, k, v, dO, alpha, wl.bq, wl.bk, rp, ci, ws=bws, out=grads, dalpha=da0)
        e[4].record()
        torch.cuda.synchronize()
        t_b = e[0].elapsed_time(e[1]) / args.steps
        t_lb = e[2].elapsed_time(e[3]) / args.steps
        bwd_flops = 10.0 * wl.bq * wl.bk * wl.d * nnz
        res["bwd"] = {"sparse_bwd_ms": t_b, "alpha_grad_ms": e[1].elapsed_time(e[2]) / args.steps,
                      "achieved": bwd_flops / (t_b * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": bwd_flops / (t_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                      "kernels": "csc_count/scan/fill + bwd_dq_kernel + bwd_dkdv_kernel",
                      "vs_sparse_fwd": t_b / t_sp,
                      # the linear branch's backward, accumulated onto the sparse
                      # branch's: mask transpose, phi tiles, the four per-head
                      # float32 products and the listed-pair row and column walks
                      "linear_bwd_ms": t_lb,
                      # the mixed output's gradient (both branches, mask
                      # transpose built once, and the alpha gradient): the
                      # training backward
                      "attn_bwd_ms": e[3].elapsed_time(e[4]) / args.steps,
                      "linear_kernels": "csc_* + lin_phi + lin_outer x2 + lin_split x3 + lin_dq + lin_dkdv"}
        # the training pair: the fused forward that also keeps each query's
        # normalisers and the two branch outputs, and the mixed backward that
        # reads them instead of recomputing them (the row kernels skip their
        # first pass)
        _, sv = S.sla_fused_fwd_save(q, k, v, alpha, wl.bq, wl.bk, rp, ci, ws, out=out)
        da = torch.empty(wl.H, dtype=torch.float32, device=dev)
        S.sla_attn_bwd_saved(q, k, v, dO, alpha, wl.bq, wl.bk, rp, ci, sv, ws=bws, out=grads, dalpha=da)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(args.steps):
            S.sla_fused_fwd_save(q, k, v, alpha, wl.bq, wl.bk, rp, ci, ws, out=out, saved=sv)
        e[1].record()
        for _ in range(args.steps):
            S.sla_attn_bwd_saved(q, k, v, dO, alpha, wl.bq, wl.bk, rp, ci, sv, ws=bws, out=grads, dalpha=da)
        e[2].record()
        torch.cuda.synchronize()
        res["bwd"]["fused_fwd_save_ms"] = e[0].elapsed_time(e[1]) / args.steps
        res["bwd"]["attn_bwd_saved_ms"] = e[1].elapsed_time(e[2]) / args.steps

    # SoftTop-k weights of every mask row (pool + logits + threshold solve),
    # the router-training form of the selection, at temperature 0.5
    if not args.no_extras:
        msoft = torch.empty((wl.B, wl.H, wl.Nq, wl.Nk), dtype=torch.float32, device=dev)
        S.sla_soft_topk(q, k, wl.bq, wl.bk, wl.k_frac, 0.5, wq, wk, out=msoft, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            S.sla_soft_topk(q, k, wl.bq, wl.bk, wl.k_frac, 0.5, wq, wk, out=msoft, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        res["soft_topk_ms"] = e0.elapsed_time(e1) / args.steps
        del msoft

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_probe_bytes"] = n * 4

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
