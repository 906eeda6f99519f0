#!/usr/bin/env python3
"""Throughput of the sparse + linear attention forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the K/V preparation pass (sla_kv_prepare, which also pools K for the mask),
the block mask (sla_mask_prepared) and the fused sparse + linear + alpha-mix
kernel (sla_fused_fwd) - the same launches as sla_attn_fwd, issued one by one
so that HIP events on the launch stream bracket each stage.  Inputs are
resident in HBM before timing starts.  The untimed warm-up runs 300 steps
(about 0.2 s): the shader clock of a GPU that was idle takes tens of
milliseconds of load to settle, and steps timed before that run 10-15%
slower.

Prints ONE JSON line.  value = dense-equivalent TFLOP/s = 4 B H N^2 d /
(time per step); the dense bf16 kernel of this library on the same tensors
gives the speedup.  The roofline object covers the fused kernel (algorithmic
FLOPs: 4 bq bk d per executed (query block, key block) pair plus 2 bq d^2 per
query block with a linear branch), the mask roofline the HBM bytes of the
standalone mask call sla_mask (Q and K read once, the CSR written once), timed
in its own leg after the steps.  cpu_baseline times the fp64
oracle on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
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
    ap.add_argument("--workload", default="video480p-sla2-N32760")
    ap.add_argument("--dense-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time spent on the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
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


def cpu_baseline(x, rows_budget_s: float):
    """The fp64 oracle as it stands on a bounded sample: the whole mask of one
    head plus the sparse and linear branches of as many of that head's query
    blocks as fit in the time budget.  Returns the dict for the JSON line."""
    import numpy as np
    from oracle import sla_oracle as O
    wl = x.wl
    q1, k1, v1 = x.Q[:1, :1], x.K[:1, :1], x.V[:1, :1]
    wq, wk = x.Wq, x.Wk
    t0 = time.perf_counter()
    rp, ci, _ = O.mask(q1, k1, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, keep_info=False)
    t_mask = time.perf_counter() - t0
    alpha = x.alpha[:1].double().numpy()
    rng = np.random.default_rng(0)
    order = rng.permutation(wl.Nq)
    n, t_rows = 0, 0.0
    while n < wl.Nq and (n < 2 or t_rows < rows_budget_s):
        i = int(order[n])
        t0 = time.perf_counter()
        O.attn(q1, k1, v1, alpha, wl.bq, wl.bk, rp, ci, rows=[(0, 0, i)])
        t_rows += time.perf_counter() - t0
        n += 1
    per_block = t_mask / wl.Nq + t_rows / n
    flops_block = 4.0 * wl.bq * wl.N * wl.d          # dense-equivalent work of one query block
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    return {"value": flops_block / per_block / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"fp64 numpy oracle on head (0,0): full mask of {wl.Nq} query blocks "
                       f"({t_mask:.2f}s) + sparse and linear branches of {n} random query blocks "
                       f"({t_rows:.2f}s); value = dense-equivalent FLOPs per query block "
                       f"(4*bq*N*d) / (mask time per block + branch time per block)"),
            "host_cpus": len(os.sched_getaffinity(0))}


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
    q, k, v, alpha = (t.to(dev).contiguous() for t in (x.Q, x.K, x.V, x.alpha))
    wq = None if x.Wq is None else x.Wq.to(dev)
    wk = None if x.Wk is None else x.Wk.to(dev)
    prob, sel = S.problem(q, wl.bq, wl.bk), S.select(wl.k_frac, wl.p, wq, wk)
    ws = S.workspace(prob, sel, dev)
    cap = S.sla_mask_capacity(prob)
    rp = torch.empty(wl.B * wl.H * wl.Nq + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(cap, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        S.sla_kv_prepare(k, v, wl.bq, wl.bk, ws, alpha)
        if ev is not None:
            ev[1].record()
        S.sla_mask_prepared(q, k, alpha, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, ws=ws, row_ptr=rp, col_idx=ci)
        if ev is not None:
            ev[2].record()
        S.sla_fused_fwd(q, k, v, alpha, wl.bq, wl.bk, rp, ci, ws, out=out)
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    st_sum = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    st_maskp = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    st_fused = sum(e[2].elapsed_time(e[3]) for e in events) / args.steps
    ev_step = sum(e[0].elapsed_time(e[3]) for e in events) / args.steps

    # the standalone mask call (pools Q and K itself), for the mask's HBM roofline
    rp_m, ci_m = torch.empty_like(rp), torch.empty_like(ci)
    mask_call = lambda: S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk, ws=ws, row_ptr=rp_m,
                                   col_idx=ci_m)
    for _ in range(10):
        mask_call()
    torch.cuda.synchronize()
    em0, em1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    em0.record()
    for _ in range(args.steps):
        mask_call()
    em1.record()
    torch.cuda.synchronize()
    st_mask = em0.elapsed_time(em1) / args.steps
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
    dense_flops = 4.0 * wl.B * wl.H * wl.N * wl.N * wl.d
    es = 2 if wl.dtype == "bf16" else 4
    mask_bytes = 2.0 * wl.B * wl.H * wl.N * wl.d * es + 4.0 * (len(counts) + 1) + 4.0 * nnz

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
                   "router": wl.router, "seed": wl.seed},
        "roofline": {"bound": "mfma", "achieved": fused_flops / (st_fused * 1e-3) / 1e12,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": fused_flops / (st_fused * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": stored_traffic(), "kernel": f"attn_kernel<d={wl.d},bq={wl.bq},bk={wl.bk},fused>",
                     "flops_per_launch": fused_flops, "ms_per_launch": st_fused},
        "mask_roofline": {"bound": "hbm", "achieved": mask_bytes / (st_mask * 1e-3) / 1e9,
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": mask_bytes / (st_mask * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "bytes_per_call": mask_bytes, "ms_per_call": st_mask},
        "stage_ms": {"kv_prepare": st_sum, "mask_prepared": st_maskp, "fused": st_fused,
                     "events_step": ev_step, "mask_standalone": st_mask},
        "sparsity": 1.0 - nnz / float(wl.B * wl.H * wl.Nq * wl.Nk), "nnz": nnz,
        "executed_TFLOPS_fused": fused_flops / (st_fused * 1e-3) / 1e12,
    }

    if not args.no_dense:
        S.sla_dense_fwd(q, k, v, wl.bq, wl.bk, out=out, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.dense_steps):
            S.sla_dense_fwd(q, k, v, wl.bq, wl.bk, out=out, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        t_dense = e0.elapsed_time(e1) / args.dense_steps
        res["dense_ms"] = t_dense
        res["dense_TFLOPS"] = dense_flops / (t_dense * 1e-3) / 1e12
        res["speedup_vs_dense"] = t_dense / ms_step

    # the sparse branch alone (sla_sparse_fwd) on this step's mask, for the
    # executed-block rate of the attention kernel
    S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci, out=out, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    t_sp = e0.elapsed_time(e1) / args.steps
    res["sparse_fwd_ms"] = t_sp
    res["sparse_fwd_executed_TFLOPS"] = pair_flops * nnz / (t_sp * 1e-3) / 1e12

    # the 8-bit sparse branch on the same mask: quantisation of Q, K, V, then
    # the two-pass int8 kernel; its algorithmic rate (4 bq bk d operations per
    # executed pair) is priced against the int8 matrix peak
    if wl.dtype == "bf16":
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

    # the sparse branch's backward (mask fixed) on this step's mask: the mask
    # transpose, the dQ pass and the dK/dV pass.  Algorithmic work: the five
    # matrix products of a softmax-attention gradient per executed pair
    # (S, dP, dV, dQ, dK: 10 bq bk d), priced against the bf16 matrix peak
    if wl.dtype == "bf16":
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
        for _ in range(args.steps):
            S.sla_attn_bwd(q, k, v, dO, alpha, wl.bq, wl.bk, rp, ci, ws=bws, out=grads)
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
                      # transpose built once): the training backward
                      "attn_bwd_ms": e[3].elapsed_time(e[4]) / args.steps,
                      "linear_kernels": "csc_* + lin_phi + lin_outer x2 + lin_split x3 + lin_dq + lin_dkdv"}

    # SoftTop-k weights of every mask row (pool + logits + threshold solve),
    # the router-training form of the selection, at temperature 0.5
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
