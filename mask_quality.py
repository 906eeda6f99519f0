#!/usr/bin/env python3
"""Synthetic mask-quality study of the hybrid block selection.

SpargeAttention2 write-up §一 and §六: Top-k keeps a fixed number of blocks
and fails on flat attention maps (too few blocks carry the mass), Top-p keeps
blocks until their mass reaches p and fails on peaked maps (it keeps almost
nothing); the union of the two covers both regimes.  This study measures that
on synthetic inputs: the routed 480p workload (its first batch entry: H 16,
N 32760, d 128, bq 128, bk 64, k_frac 0.03) with the query temperature tau in {0.25, 1, 4}
(flat to peaked pooled maps) and p in {0.3, 0.6, 0.9}.  For each setting it
builds three masks - Top-k alone (p = 0), Top-p alone (k_frac = 0) and the
union - and reports the fraction of blocks kept and the attention mass the
kept blocks capture: on the pooled block map (sum of the selected blocks'
pooled probabilities, the quantity Top-p targets) and at token level (the
exact softmax of every query over all N keys, summed over the keys of the
selected blocks, on sampled query blocks) - and the relative L1 error of the
sparse branch's output against dense attention.  That error is reported but is
a weak signal on these inputs: with V ~ N(0, 1) independent of the scores the
dense output averages ~N random rows and the sparse one ~n_sel * bk rows, so
their difference is mostly that norm mismatch; dense O = m * O_s + (1 - m) *
O_rest with m the captured token mass, so 1 - m is what the mask controls.

Everything runs on the library's GPU kernels (mask, sparse branch, dense);
no weights or datasets are involved.  Prints one JSON line per (tau, p) and a
markdown table.  Usage: python mask_quality.py [--heads H] [--samples S]
"""
from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def rule_stats(S, q, k, wl, wq, wk, k_frac: float, p: float, samples):
    """One selection rule (k_frac, p) on one head set: the library's mask and
    the quantities of the study.  q, k [1, H, N, d] on the GPU; samples: the
    (head, query block) pairs of the token-level mass.  Returns (row_ptr,
    col_idx, stats) with stats = kept (fraction of blocks selected),
    pooled_mass (mean over rows of the selected blocks' pooled
    probabilities) and token_mass (mean over the sampled blocks' queries of
    the exact softmax mass on the selected keys)."""
    import torch
    H, N, d = q.shape[1], q.shape[2], q.shape[3]
    R = H * wl.Nq
    rp, ci, logits = S.sla_mask(q, k, wl.bq, wl.bk, k_frac, p, wq, wk, return_logits=True)
    torch.cuda.synchronize()
    rp_h, ci_h = rp.cpu().long(), ci.cpu().long()
    P = torch.softmax(logits.reshape(R, wl.Nk), dim=-1).cpu()
    pooled = 0.0
    for r in range(R):
        pooled += P[r, ci_h[rp_h[r]:rp_h[r + 1]]].sum().item()
    token = 0.0
    for (h, i) in samples:
        r = h * wl.Nq + i
        sel = ci_h[rp_h[r]:rp_h[r + 1]]
        keep = torch.zeros(N, dtype=torch.bool, device=q.device)
        for j in sel.tolist():
            keep[j * wl.bk:min((j + 1) * wl.bk, N)] = True
        qi = q[0, h, i * wl.bq:min((i + 1) * wl.bq, N)].float()
        a = torch.softmax(qi @ k[0, h].float().T / d ** 0.5, dim=-1)
        token += a[:, keep].sum(dim=-1).mean().item()
    stats = {"kept": int(rp_h[-1]) / (R * wl.Nk), "pooled_mass": pooled / R,
             "token_mass": token / max(len(samples), 1)}
    return rp, ci, stats


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--heads", type=int, default=16, help="heads of the first batch entry to generate")
    ap.add_argument("--samples", type=int, default=4, help="query blocks per head for the token-level mass")
    args = ap.parse_args()
    import torch

    import block_sparse_linear_sla_amd as S
    import gen

    if not torch.cuda.is_available():
        print("mask_quality.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    base = gen.WORKLOADS["video480p-router-N32760"]
    dev = torch.device("cuda:0")
    gsel = torch.Generator().manual_seed(0)
    rows = []
    for tau in gen.ROUTER_TAUS:
        wl = base.with_(tau=tau)
        x = gen.make(wl, heads=args.heads)
        q, k, v = (t.to(dev).contiguous() for t in (x.Q, x.K, x.V))
        wq, wk = x.Wq.to(dev), x.Wk.to(dev)
        H = q.shape[1]
        od = S.sla_dense_fwd(q, k, v, wl.bq, wl.bk)
        od_l1 = od.float().abs().sum().item()
        samp = [(h, int(i)) for h in range(H) for i in torch.randperm(wl.Nq, generator=gsel)[:args.samples]]
        for p in (0.3, 0.6, 0.9):
            res = {"tau": tau, "p": p, "k_frac": wl.k_frac}
            for rule, kf, pp in (("topk", wl.k_frac, 0.0), ("topp", 0.0, p), ("union", wl.k_frac, p)):
                rp, ci, st = rule_stats(S, q, k, wl, wq, wk, kf, pp, samp)
                os_ = S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci)
                res[f"{rule}_rel_l1"] = (os_.float() - od.float()).abs().sum().item() / od_l1
                for key, val in st.items():
                    res[f"{rule}_{key}"] = val
            rows.append(res)
            print(json.dumps(res), flush=True)
    print("\n| tau | p | Top-k: kept / pooled / token mass / rel-L1 | Top-p: kept / pooled / token mass "
          "/ rel-L1 | union: kept / pooled / token mass / rel-L1 |")
    print("|---|---|---|---|---|")
    for r in rows:
        cells = [f"{r[f'{u}_kept']:.3f} / {r[f'{u}_pooled_mass']:.3f} / {r[f'{u}_token_mass']:.3f}"
                 f" / {r[f'{u}_rel_l1']:.2f}"
                 for u in ("topk", "topp", "union")]
        print(f"| {r['tau']} | {r['p']} | " + " | ".join(cells) + " |")


if __name__ == "__main__":
    main()
