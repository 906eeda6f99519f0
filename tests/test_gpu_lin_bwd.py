"""GPU parity of the linear-branch backward against the oracle (float64
autograd of the linear branch over each row block's unselected keys, mask
fixed).

Bar, derived from the arithmetic: the kernels take bf16 inputs exactly,
form phi(Q) and phi(K) once as bf16 matrix-core operands (relative 2^-9),
keep the per-head totals and per-query terms in float32, round the
listed-pair weights to bf16 where they enter a matrix product (2^-9) and the
outputs to bf16 (2^-9; once more when accumulating).  These roundings are
independent from element to element, so, as for the sparse branch, each
gradient tensor must stay within a relative L1 error of 1e-2 of the exact one
and every element within 2e-2 of the tensor's largest magnitude.

At the 480p workload's full length the oracle differentiates sampled row
blocks (their dQ rows are exact), and two identities that hold at any size
check the rest: dV summed over keys equals dO_l summed over the rows that
have a linear branch, and rescaling phi(k) for all keys (phi(q_t) for one
query) leaves O_l unchanged, so sum_u phi(k_u) . dphi(k_u) = 0 per head and
phi(q_t) . dphi(q_t) = 0 per query, with dphi = grad / phi'."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U
from tests.test_gpu_bwd import _compare, _random_csr, _skewed_csr

pytestmark = pytest.mark.gpu


def _inputs(x, rp, ci, seed):
    q, k, v = U.dev(x.Q, x.K, x.V)
    dO = torch.from_numpy(np.random.default_rng(seed).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    rpt = torch.from_numpy(rp).int().cuda()
    cit = torch.from_numpy(ci).int().cuda() if len(ci) else torch.zeros(1, dtype=torch.int32, device="cuda")
    return q, k, v, dO, rpt, cit


CASES = [
    # name, N, d, bq, bk, density
    ("ragged-1000", 1000, 128, 128, 64, 0.3),
    ("d64-bq64-bk128-777", 777, 64, 64, 128, 0.4),
    ("bq64-bk128-1500", 1500, 128, 64, 128, 0.25),
    ("d64-600", 600, 64, 128, 64, 0.5),
    ("sparse-2100", 2100, 128, 128, 64, 0.05),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_bwd_small(case):
    name, N, d, bq, bk, density = case
    print(f"[lin-bwd] {name}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=23)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    # row 1 lists nothing (linear over every key), the last row lists every
    # block (no linear branch)
    rp, ci = _random_csr(np.random.default_rng(11), 2, Nq, Nk, density, empty_rows={1},
                         full_rows={2 * Nq - 1})
    q, k, v, dO, rpt, cit = _inputs(x, rp, ci, seed=6)
    dq, dk, dv = S.sla_linear_bwd(q, k, v, dO.cuda(), bq, bk, rpt, cit)
    torch.cuda.synchronize()
    ref = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    _compare(dq, ref["dQ"], "dQ")
    _compare(dk, ref["dK"], "dK")
    _compare(dv, ref["dV"], "dV")
    # the fully listed row block has no linear branch: its dQ rows are 0
    s0 = (Nq - 1) * bq
    assert not dq[0, 1, s0:].any()


@pytest.mark.parametrize("bk", [64, 128])
def test_linear_bwd_skewed_columns(bk):
    """Key blocks listed by every row, by half of them, by about 10% and by
    none (the column kernel's launch order across its classes)."""
    N, d, bq = 4000, 128, 128
    print(f"[lin-bwd] skewed columns bk={bk}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=37)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _skewed_csr(np.random.default_rng(14), 2, Nq, Nk)
    q, k, v, dO, rpt, cit = _inputs(x, rp, ci, seed=10)
    dq, dk, dv = S.sla_linear_bwd(q, k, v, dO.cuda(), bq, bk, rpt, cit)
    torch.cuda.synchronize()
    ref = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    _compare(dq, ref["dQ"], "dQ")
    _compare(dk, ref["dK"], "dK")
    _compare(dv, ref["dV"], "dV")


def test_linear_bwd_accumulates_onto_sparse():
    """Both branches into one set of buffers: sparse branch's gradient with
    alpha dO, then the linear branch's with (1 - alpha) dO added."""
    N, d, bq, bk, alpha = 900, 128, 128, 64, 0.7
    print(f"[lin-bwd] accumulate N={N}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=29)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(12), 2, Nq, Nk, 0.35)
    q, k, v, dO, rpt, cit = _inputs(x, rp, ci, seed=7)
    g = dO.cuda()
    gs = (alpha * g.float()).to(torch.bfloat16)
    gl = ((1 - alpha) * g.float()).to(torch.bfloat16)
    ws = S.bwd_workspace(S.problem(q, bq, bk), q.device)
    out = S.sla_sparse_bwd(q, k, v, gs, bq, bk, rpt, cit, ws=ws)
    S.sla_linear_bwd(q, k, v, gl, bq, bk, rpt, cit, ws=ws, out=out, accumulate=True)
    torch.cuda.synchronize()
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, gs.cpu())
    rl = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, gl.cpu())
    for t, n in zip(out, ("dQ", "dK", "dV")):
        _compare(t, rs[n] + rl[n], n)


def _dphi_inv(x):
    """1 / phi'(x) for phi = elu + 1, float64."""
    return np.where(x > 0, 1.0, np.exp(-np.minimum(x, 0.0)))


def test_linear_bwd_480p_two_heads():
    """The 480p SLA2 workload at full length (N = 32760) on two heads with the
    library's own mask: sampled row blocks against the oracle, identities for
    the rest."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[lin-bwd] {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k, v = U.dev(x.Q, x.K, x.V)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    dO = torch.from_numpy(np.random.default_rng(8).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    dq, dk, dv = S.sla_linear_bwd(q, k, v, dO.cuda(), wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    B, H, N, d = x.Q.shape
    Nq = O.n_blocks(N, wl.bq)
    rows = [(0, 0, 0), (0, 0, Nq // 2), (0, 1, 77), (0, 1, Nq - 1)]
    ref = O.linear_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    for (b, h, i) in rows:
        s, e = i * wl.bq, min(N, (i + 1) * wl.bq)
        _compare(dq[b, h, s:e], ref["dQ"][b, h, s:e], f"dQ rows of block {i}, head {h}")
    _linear_identities(x, wl, rp, dO, dq, dk, dv)


def _linear_identities(x, wl, rp, dO, dq, dk, dv):
    """Every key and query of every head: dV sums to dO_l over the rows with a
    linear branch, sum_u phi(k_u) . dphi(k_u) = 0 per head and phi(q_t) .
    dphi(q_t) = 0 per query."""
    B, H, N, d = x.Q.shape
    Nq = O.n_blocks(N, wl.bq)
    Qd, Kd = O.as_f64(x.Q), O.as_f64(x.K)
    G = O.as_f64(dO)
    dqd, dkd, dvd = (t.cpu().double().numpy() for t in (dq, dk, dv))
    for h in range(H):
        # dV sums to dO over the rows with a linear branch
        has = np.zeros(N, dtype=bool)
        for i in range(Nq):
            r = h * Nq + i
            if rp[r + 1] - rp[r] < O.n_blocks(N, wl.bk):
                has[i * wl.bq:(i + 1) * wl.bq] = True
        want = G[0, h][has].sum(0)
        got = dvd[0, h].sum(0)
        scale = np.abs(G[0, h][has]).sum(0).max()
        err = np.abs(got - want).max() / scale
        print(f"  head {h}: sum dV vs sum dO_l: {err:.3g} of sum|dO_l|")
        assert err <= 1e-2
        # sum_u phi(k_u) . dphi(k_u) = 0
        pk = O.phi(Kd[0, h])
        terms = pk * dkd[0, h] * _dphi_inv(Kd[0, h])
        rel = abs(terms.sum()) / np.abs(terms).sum()
        print(f"  head {h}: sum phi(k) . dphi(k): {rel:.3g} of sum |terms|")
        assert rel <= 1e-2
        # phi(q_t) . dphi(q_t) = 0 per query
        pq = O.phi(Qd[0, h])
        tq = pq * dqd[0, h] * _dphi_inv(Qd[0, h])
        relq = np.abs(tq.sum(1)) / np.maximum(np.abs(tq).sum(1), 1e-30)
        print(f"  head {h}: per-query phi(q) . dphi(q): max {relq.max():.3g}, mean {relq.mean():.3g}")
        assert relq.mean() <= 2e-2


def test_linear_bwd_720p_one_head():
    """The 720p SLA2 workload at full length (N = 75600, 591 x 1182 blocks) on
    one head with the library's mask: sampled row blocks (the longest and
    shortest rows, the middle and the ragged last) against the oracle, the
    identities for every key and query."""
    wl = gen.WORKLOADS["video720p-sla2-N75600"]
    print(f"[lin-bwd] {wl.name}, 1 head", flush=True)
    x = gen.make(wl, heads=1)
    q, k, v = U.dev(x.Q, x.K, x.V)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    dO = torch.from_numpy(np.random.default_rng(16).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    dq, dk, dv = S.sla_linear_bwd(q, k, v, dO.cuda(), wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    N = x.Q.shape[2]
    counts = np.diff(rp)
    Nq = len(counts)
    rows = sorted({(0, 0, int(np.argmax(counts))), (0, 0, int(np.argmin(counts))), (0, 0, 137),
                   (0, 0, Nq // 2), (0, 0, Nq - 1)})
    ref = O.linear_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    for (b, h, i) in rows:
        s, e = O.block_range(i, wl.bq, N)
        _compare(dq[b, h, s:e], ref["dQ"][b, h, s:e], f"dQ rows of block {i}")
    _linear_identities(x, wl, rp, dO, dq, dk, dv)


@pytest.mark.parametrize("N,d,bq,bk", [(1000, 128, 128, 64), (777, 64, 64, 128)])
def test_attn_bwd_mixed(N, d, bq, bk):
    """sla_attn_bwd: alpha_h times the sparse branch's gradient plus
    (1 - alpha_h) times the linear branch's, both taken with dO, on four heads
    whose ratios include the two ends (alpha = 1: sparse only; 0: linear only)."""
    print(f"[lin-bwd] mixed N={N} d={d} bq={bq} bk={bk}", flush=True)
    H = 4
    wl = gen.Workload("adhoc", B=1, H=H, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=31)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(13), H, Nq, Nk, 0.3, empty_rows={2},
                         full_rows={H * Nq - 1})
    q, k, v, dO, rpt, cit = _inputs(x, rp, ci, seed=9)
    alpha = torch.tensor([0.7, 1.0, 0.0, 0.35], dtype=torch.float32)
    da = torch.full((H,), float("nan"), dtype=torch.float32, device="cuda")
    dq, dk, dv = S.sla_attn_bwd(q, k, v, dO.cuda(), alpha.cuda(), bq, bk, rpt, cit, dalpha=da)
    torch.cuda.synchronize()
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    a = alpha.double().numpy()[None, :, None, None]
    for t, n in zip((dq, dk, dv), ("dQ", "dK", "dV")):
        _compare(t, a * rs[n] + (1 - a) * rl[n], n)
        # the alpha = 1 head carries the sparse branch's gradient alone, the
        # alpha = 0 head the linear branch's alone
        _compare(t[:, 1:2], rs[n][:, 1:2], n + " (alpha 1)")
        _compare(t[:, 2:3], rl[n][:, 2:3], n + " (alpha 0)")
    # the alpha gradient from the row kernels' per-query terms, every head
    # (the ends included: both branches' terms are formed whatever alpha is)
    Os = O.assemble(O.sparse_branch(x.Q, x.K, x.V, bq, bk, rp, ci), 1, H, N, d, bq)
    Ol = O.assemble(O.linear_branch(x.Q, x.K, x.V, bq, bk, rp, ci), 1, H, N, d, bq)
    exact = O.alpha_grad(dO, Os, Ol)
    scale = (np.abs(O.as_f64(dO)) * (np.abs(Os) + np.abs(Ol))).sum(axis=(0, 2, 3))
    got = da.cpu().double().numpy()
    print(f"  dalpha {got}, exact {exact}")
    assert np.all(np.abs(got - exact) <= 1e-4 * scale), (got, exact)


def test_attn_bwd_480p_two_heads():
    """sla_attn_bwd on the 480p workload at full length (two heads, the
    library's mask, the workload's alpha): dQ of sampled row blocks against
    alpha times the oracle's sparse-branch gradient plus (1 - alpha) times its
    linear-branch gradient; and, since every row has both branches there,
    dV summed over the keys equals dO summed over the queries (each branch's
    weights over its keys sum to one)."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[lin-bwd] sla_attn_bwd {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k, v = U.dev(x.Q, x.K, x.V)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    dO = torch.from_numpy(np.random.default_rng(10).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    alpha = x.alpha.float()
    dq, dk, dv = S.sla_attn_bwd(q, k, v, dO.cuda(), alpha.cuda(), wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    B, H, N, d = x.Q.shape
    Nq, Nk = O.n_blocks(N, wl.bq), O.n_blocks(N, wl.bk)
    counts = np.diff(rp)
    assert counts.min() > 0 and counts.max() < Nk  # both branches on every row
    rows = [(0, 0, 3), (0, 1, Nq - 1)]
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    a = alpha.double().numpy()
    for (b, h, i) in rows:
        s, e = i * wl.bq, min(N, (i + 1) * wl.bq)
        ref = a[h] * rs["dQ"][b, h, s:e] + (1 - a[h]) * rl["dQ"][b, h, s:e]
        _compare(dq[b, h, s:e], ref, f"dQ rows of block {i}, head {h}")
    G = O.as_f64(dO)
    dvd = dv.cpu().double().numpy()
    for h in range(H):
        err = np.abs(dvd[0, h].sum(0) - G[0, h].sum(0)).max() / np.abs(G[0, h]).sum(0).max()
        print(f"  head {h}: sum dV vs sum dO: {err:.3g} of sum|dO|")
        assert err <= 1e-2


def test_attn_bwd_two_batches():
    """B = 2: the (b, h) slices of every kernel of the backward (the mask
    transpose, the row and column walks, the per-head totals) index past the
    first batch."""
    N, d, bq, bk = 700, 64, 64, 64
    print(f"[lin-bwd] mixed B=2 N={N}", flush=True)
    wl = gen.Workload("adhoc", B=2, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, alpha=(0.8, 0.4), seed=37)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(14), 4, Nq, Nk, 0.3, empty_rows={5},
                         full_rows={4 * Nq - 1})
    q, k, v, dO, rpt, cit = _inputs(x, rp, ci, seed=11)
    alpha = torch.tensor([0.8, 0.4], dtype=torch.float32)
    dq, dk, dv = S.sla_attn_bwd(q, k, v, dO.cuda(), alpha.cuda(), bq, bk, rpt, cit)
    torch.cuda.synchronize()
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    a = alpha.double().numpy()[None, :, None, None]
    for t, n in zip((dq, dk, dv), ("dQ", "dK", "dV")):
        _compare(t, a * rs[n] + (1 - a) * rl[n], n)
        _compare(t[1:], (a * rs[n] + (1 - a) * rl[n])[1:], n + " (second batch)")


def test_attn_bwd_bitwise_deterministic():
    """The mixed backward at the 480p length (two heads, the library's mask):
    two calls, the second on a workspace filled with 0xff bytes first, give
    the same dQ, dK, dV and alpha gradient bit for bit (the column kernels'
    launch order comes from LDS atomics and may differ between runs; every
    sum still runs in a fixed order).  The same for the saved-terms call."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[lin-bwd] determinism {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    rp, ci = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    g = torch.from_numpy(np.random.default_rng(21).normal(size=tuple(x.Q.shape))).to(torch.bfloat16).cuda()
    prob = S.problem(q, wl.bq, wl.bk)
    ws = S.workspace(prob, S.select(wl.k_frac, wl.p), q.device)
    S.sla_kv_prepare(k, v, wl.bq, wl.bk, ws, a)
    _, sv = S.sla_fused_fwd_save(q, k, v, a, wl.bq, wl.bk, rp, ci, ws)
    outs = []
    for fill in (None, 0xFF):
        bws = S.bwd_workspace(prob, q.device)
        if fill is not None:
            bws.fill_(fill)
        da = torch.empty(2, dtype=torch.float32, device="cuda")
        r = S.sla_attn_bwd(q, k, v, g, a, wl.bq, wl.bk, rp, ci, ws=bws, dalpha=da) + (da,)
        bws.fill_(0xFF)
        r2 = S.sla_attn_bwd_saved(q, k, v, g, a, wl.bq, wl.bk, rp, ci, sv, ws=bws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in r + r2])
    names = ("dQ", "dK", "dV", "dalpha", "saved dQ", "saved dK", "saved dV", "saved dalpha")
    for n, t0, t1 in zip(names, outs[0], outs[1]):
        assert torch.equal(t0, t1), f"{n} differs between runs"
