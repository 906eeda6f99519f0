"""Helpers shared by the GPU parity tests: device transfer, the oracle run
per head (to bound host memory), the cut-off rule for masks, error metrics."""
from __future__ import annotations

import numpy as np
import torch

import gen
from oracle import sla_oracle as O

_ROUTER_X = {}


def router_inputs(tau):
    """Inputs of the routed 480p workload at query temperature tau, generated
    once and kept (one temperature at a time: the sweeps run tau-major, so
    host memory holds one set)."""
    if tau not in _ROUTER_X:
        _ROUTER_X.clear()
        _ROUTER_X[tau] = gen.make(gen.WORKLOADS["video480p-router-N32760"].with_(tau=tau))
    return _ROUTER_X[tau]


def has_gpu() -> bool:
    return torch.cuda.is_available()


def dev(*ts):
    return tuple(None if t is None else t.to("cuda").contiguous() for t in ts)


def csr(rp: torch.Tensor, ci: torch.Tensor):
    rp = rp.to("cpu").numpy().astype(np.int64)
    ci = ci.to("cpu").numpy()[: rp[-1]].astype(np.int64)
    return rp, ci


def oracle_mask_per_head(x, k_frac, p, keep_info=True):
    """oracle.mask run one (b, h) at a time and concatenated (rows (b, h, i))."""
    B, H = x.Q.shape[:2]
    rps, cis, S, P, rows = [], [], [], [], []
    off = 0
    k = None
    for b in range(B):
        for h in range(H):
            rp, ci, meta = O.mask(x.Q[b:b + 1, h:h + 1], x.K[b:b + 1, h:h + 1], x.wl.bq, x.wl.bk,
                                  k_frac, p, x.Wq, x.Wk, keep_info=keep_info)
            rps.append(rp[1:] + off)
            off += rp[-1]
            cis.append(ci)
            S.append(meta["S"][0, 0])
            P.append(meta["P"][0, 0])
            rows.extend(meta["rows"])
            k = meta["k"]
    rp = np.concatenate([[0]] + rps).astype(np.int64)
    ci = np.concatenate(cis).astype(np.int64)
    return rp, ci, dict(S=np.stack(S), P=np.stack(P), rows=rows, k=k)


def mask_mismatches(rp_g, ci_g, rp_o, ci_o, meta, p, tol=1e-5):
    """Blocks where the GPU and oracle masks differ and that are NOT excused.

    A differing block is excused when (i) its pooled logit lies within tol of
    the logit at the oracle's last kept position, or (ii) an oracle cumulative
    mass next to it in the oracle order (just before or just after it) lies
    within tol of p (the Top-p cut lives in cumulative-mass space).
    Returns (unexcused list of (row, block), excused count, differing rows)."""
    S = meta["S"].reshape(-1, meta["S"].shape[-1])
    p64 = float(np.float32(p))
    bad, excused, rows = [], 0, 0
    for r in range(len(rp_o) - 1):
        g = set(ci_g[rp_g[r]:rp_g[r + 1]].tolist())
        o = set(ci_o[rp_o[r]:rp_o[r + 1]].tolist())
        if g == o:
            continue
        rows += 1
        info = meta["rows"][r]
        order, cum, n = info["order"], info["cum"], info["n"]
        rank = np.empty_like(order)
        rank[order] = np.arange(len(order))
        thr = S[r, order[n - 1]] if n > 0 else S[r, order[0]]
        for j in g ^ o:
            rj = rank[j]
            before = cum[rj - 1] if rj > 0 else 0.0
            after = cum[rj]
            ok = abs(S[r, j] - thr) <= tol or abs(before - p64) <= tol or abs(after - p64) <= tol
            if ok:
                excused += 1
            else:
                bad.append((r, int(j)))
    return bad, excused, rows


def check_csr_structure(rp, ci, R, Nk):
    assert rp[0] == 0 and len(rp) == R + 1
    assert np.all(np.diff(rp) >= 0)
    for r in range(R):
        row = ci[rp[r]:rp[r + 1]]
        assert np.all(row >= 0) and np.all(row < Nk)
        assert np.all(np.diff(row) > 0), f"row {r} not strictly ascending"


def errors(got: np.ndarray, ref: np.ndarray):
    """(max-abs, relative L1 = sum|got-ref| / sum|ref|)."""
    d = np.abs(got - ref)
    return float(d.max()), float(d.sum() / max(np.abs(ref).sum(), 1e-300))


def rows_of(out: torch.Tensor, rows, bq: int) -> dict:
    """Slice GPU output [B, H, N, d] into {(b, h, i): block rows} as float64."""
    N = out.shape[2]
    res = {}
    for (b, h, i) in rows:
        s, e = O.block_range(i, bq, N)
        res[(b, h, i)] = out[b, h, s:e].to("cpu", torch.float64).numpy()
    return res


def compare_rows(got: dict, ref: dict):
    g = np.concatenate([got[k].ravel() for k in sorted(ref)])
    r = np.concatenate([ref[k].ravel() for k in sorted(ref)])
    return errors(g, r)


def xcd_ranges(R, nx=8):
    """The contiguous mask-row range [start, end) each of the nx XCDs walks
    under the attention kernels' workgroup-to-row mapping: the first R % nx
    ranges hold R // nx + 1 rows, the others R // nx."""
    q, r = divmod(R, nx)
    out, start = [], 0
    for x in range(nx):
        n = q + 1 if x < r else q
        out.append((start, start + n))
        start += n
    return out


def pick_rows(rp, B, H, Nq, n=32, seed=0, heads=4):
    """At least n mask rows (b, h, i) chosen to expose indexing mistakes:
    the longest and the shortest row (most / fewest listed blocks), the
    partial last query block of the first, the last and `heads` random
    heads, the first and the last row of every XCD's range, then random
    rows up to n."""
    rng = np.random.default_rng(seed)
    counts = np.diff(np.asarray(rp, dtype=np.int64))
    R = B * H * Nq
    assert len(counts) == R
    rs = {int(np.argmax(counts)), int(np.argmin(counts)),
          int(len(counts) - 1 - np.argmax(counts[::-1])), int(len(counts) - 1 - np.argmin(counts[::-1]))}
    hs = {0, B * H - 1} | {int(v) for v in rng.integers(0, B * H, size=heads)}
    rs |= {bh * Nq + Nq - 1 for bh in hs}
    for a, e in xcd_ranges(R):
        if e > a:
            rs |= {a, e - 1}
    while len(rs) < n:
        rs.add(int(rng.integers(R)))
    return sorted((r // (H * Nq), (r // Nq) % H, r % Nq) for r in rs)


def sample_rows(B, H, Nq, n, seed=0):
    """A few (b, h, i) rows: always the first and the (possibly partial) last
    query block, plus random ones."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, 0), (B - 1, H - 1, Nq - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Nq))))
    return sorted(rows)
