"""The training pair sla_fused_fwd_save / sla_attn_bwd_saved.

The forward must give sla_fused_fwd's output bit for bit and keep: each
query's log2 sparse-branch normaliser (the oracle's log-normaliser times
log2 e, +inf for a row with no listed block), the inverse linear-branch
denominator (0 where the row has no linear branch), and the two branch
outputs (the oracle's branches at the bf16 bar; the sparse branch on every
head, the linear branch 0 on a head whose alpha is exactly 1, whose totals
the preparation pass skips).  The backward that reads
them must meet the same bar as sla_attn_bwd against the oracle's
alpha-weighted branch gradients.

Bars.  lse2: the kernel sums bf16-rounded probabilities (8 significant bits:
relative error at most 2^-8 each, round-to-nearest) relative to its running
maximum, so log2 of the sum is off by at most log2(1 + 2^-8) < 5.7e-3 (6e-3
allowed for the float32 scores);
invden: the denominator subtracts the listed keys' bf16 phi(k) sums from a
float32 total, relative 5e-3 allowed."""
import math

import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U
from tests.test_gpu_bwd import _compare, _random_csr

pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


def _forward(x, rp, ci, alpha):
    wl = x.wl
    q, k, v = U.dev(x.Q, x.K, x.V)
    a = alpha.cuda()
    rpt = torch.from_numpy(rp).int().cuda()
    cit = torch.from_numpy(ci).int().cuda() if len(ci) else torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = S.workspace(S.problem(q, wl.bq, wl.bk), S.select(wl.k_frac, wl.p), q.device)
    S.sla_kv_prepare(k, v, wl.bq, wl.bk, ws, a)
    o_plain = S.sla_fused_fwd(q, k, v, a, wl.bq, wl.bk, rpt, cit, ws)
    o, sv = S.sla_fused_fwd_save(q, k, v, a, wl.bq, wl.bk, rpt, cit, ws)
    torch.cuda.synchronize()
    return (q, k, v, a, rpt, cit), o_plain, o, sv


def _check_saved(x, rp, ci, alpha, sv, rows):
    wl = x.wl
    B, H, N, d = x.Q.shape
    Nq, Nk = O.n_blocks(N, wl.bq), O.n_blocks(N, wl.bk)
    lse = sv["lse2"].cpu().numpy().reshape(B * H * Nq, wl.bq)
    inv = sv["invden"].cpu().numpy().reshape(B * H * Nq, wl.bq)
    ref_lse = O.sparse_branch_lse(x.Q, x.K, wl.bq, wl.bk, rp, ci, rows)
    ref_den = O.linear_branch_den(x.Q, x.K, wl.bq, wl.bk, rp, ci, rows)
    ref_s = O.sparse_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, rows)
    ref_l = O.linear_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, rows)
    worst_l, worst_d = 0.0, 0.0
    for (b, h, i) in rows:
        r = (b * H + h) * Nq + i
        s, e = O.block_range(i, wl.bq, N)
        n = e - s
        a = float(alpha[h])
        listed = rp[r + 1] - rp[r]
        if listed == 0:
            assert np.all(lse[r, :n] == np.inf), f"row {r}: expected +inf"
        else:
            err = np.abs(lse[r, :n] - ref_lse[(b, h, i)] * LOG2E).max()
            worst_l = max(worst_l, err)
            assert err <= 6e-3, (r, err)
        if a == 1.0 or listed == Nk:
            assert np.all(inv[r, :n] == 0.0), f"row {r}: expected 0"
        else:
            rel = np.abs(inv[r, :n] * ref_den[(b, h, i)] - 1.0).max()
            worst_d = max(worst_d, rel)
            assert rel <= 5e-3, (r, rel)
        assert np.all(lse[r, n:] == np.inf) and np.all(inv[r, n:] == 0.0), f"row {r}: entries past N"
    print(f"  lse2: worst |err| {worst_l:.3g}; invden: worst relative err {worst_d:.3g}")
    # the linear branch of a head whose alpha is exactly 1 is not computed
    ref_l = {r: (ref_l[r] if float(alpha[r[1]]) != 1.0 else 0.0 * ref_l[r]) for r in ref_l}
    for key, got, ref in (("O_s", sv["o_s"], ref_s), ("O_l", sv["o_l"], ref_l)):
        m, rel = U.compare_rows(U.rows_of(got, rows, wl.bq), ref)
        print(f"  {key}: max-abs {m:.3g} rel {rel:.3g}")
        assert m <= 2e-2 and rel <= 5e-3, (key, m, rel)


SMALL = [
    # N, d, bq, bk, B
    (1000, 128, 128, 64, 1),
    (777, 64, 64, 128, 1),
    (1500, 128, 64, 64, 1),
    (900, 64, 128, 128, 2),
]


@pytest.mark.parametrize("N,d,bq,bk,B", SMALL)
def test_saved_forward_and_backward_small(N, d, bq, bk, B):
    """Four heads with alpha 0.7, 1, 0, 0.35 (both ends), an empty row and a
    fully listed row: every row of the forward's terms and the backward's
    every element against the oracle."""
    print(f"[saved] N={N} d={d} bq={bq} bk={bk} B={B}", flush=True)
    H = 4
    wl = gen.Workload("adhoc", B=B, H=H, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=31)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(13), B * H, Nq, Nk, 0.3, empty_rows={2, 5},
                         full_rows={B * H * Nq - 1})
    alpha = torch.tensor([0.7, 1.0, 0.0, 0.35], dtype=torch.float32)
    (q, k, v, a, rpt, cit), o_plain, o, sv = _forward(x, rp, ci, alpha)
    assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16)), "O differs from sla_fused_fwd's"
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(Nq)]
    _check_saved(x, rp, ci, alpha.numpy(), sv, rows)
    dO = torch.from_numpy(np.random.default_rng(9).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    dq, dk, dv, da = S.sla_attn_bwd_saved(q, k, v, dO.cuda(), a, bq, bk, rpt, cit, sv)
    torch.cuda.synchronize()
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    w = alpha.double().numpy()[None, :, None, None]
    for t, n in zip((dq, dk, dv), ("dQ", "dK", "dV")):
        _compare(t, w * rs[n] + (1 - w) * rl[n], n)
        _compare(t[:, 1:2], rs[n][:, 1:2], n + " (alpha 1)")
        _compare(t[:, 2:3], rl[n][:, 2:3], n + " (alpha 0)")
    # the alpha gradient: the float64 sum over the kept float32 outputs, and
    # against the oracle's branches (the alpha = 1 head has no O_l)
    G = O.as_f64(dO)
    os_, ol_ = sv["o_s"].cpu().double().numpy(), sv["o_l"].cpu().double().numpy()
    got = da.cpu().double().numpy()
    want = (G * (os_ - ol_)).sum(axis=(0, 2, 3))
    assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max(), (got, want)
    Os_ref = O.assemble(O.sparse_branch(x.Q, x.K, x.V, bq, bk, rp, ci), B, H, N, d, bq)
    Ol_ref = O.assemble(O.linear_branch(x.Q, x.K, x.V, bq, bk, rp, ci), B, H, N, d, bq)
    exact = (G * (Os_ref - Ol_ref)).sum(axis=(0, 2, 3))
    scale = (np.abs(G) * (np.abs(Os_ref) + np.abs(Ol_ref))).sum(axis=(0, 2, 3))
    print(f"  dalpha {got}, exact {exact}")
    for h in (0, 2, 3):
        assert abs(got[h] - exact[h]) <= 2e-3 * scale[h], (h, got[h], exact[h])


def test_saved_480p_two_heads():
    """The 480p SLA2 workload at full length on two heads with the library's
    mask and the workload's alpha: the forward's terms on sampled rows, the
    backward's dQ on sampled row blocks against the oracle and against
    sla_attn_bwd, and sum dV = sum dO over every key."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[saved] {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k = U.dev(x.Q, x.K)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    alpha = x.alpha.float()
    (q, k, v, a, rpt, cit), o_plain, o, sv = _forward(x, rp, ci, alpha)
    assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16)), "O differs from sla_fused_fwd's"
    B, H, N, d = x.Q.shape
    Nq = O.n_blocks(N, wl.bq)
    rows = U.pick_rows(rp, B, H, Nq, n=12, seed=4)
    _check_saved(x, rp, ci, alpha.numpy(), sv, rows)
    dO = torch.from_numpy(np.random.default_rng(10).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    g = dO.cuda()
    dq, dk, dv, da = S.sla_attn_bwd_saved(q, k, v, g, a, wl.bq, wl.bk, rpt, cit, sv)
    dq0, dk0, dv0 = S.sla_attn_bwd(q, k, v, g, a, wl.bq, wl.bk, rpt, cit)
    torch.cuda.synchronize()
    for t, t0, n in zip((dq, dk, dv), (dq0, dk0, dv0), ("dQ", "dK", "dV")):
        _compare(t, t0.cpu().double().numpy(), n + " against sla_attn_bwd")
    drows = [(0, 0, 3), (0, 1, Nq - 1)]
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=drows)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=drows)
    w = alpha.double().numpy()
    for (b, h, i) in drows:
        s, e = O.block_range(i, wl.bq, N)
        _compare(dq[b, h, s:e], w[h] * rs["dQ"][b, h, s:e] + (1 - w[h]) * rl["dQ"][b, h, s:e],
                 f"dQ rows of block {i}, head {h}")
    G = O.as_f64(dO)
    dvd = dv.cpu().double().numpy()
    for h in range(H):
        err = np.abs(dvd[0, h].sum(0) - G[0, h].sum(0)).max() / np.abs(G[0, h]).sum(0).max()
        print(f"  head {h}: sum dV vs sum dO: {err:.3g} of sum|dO|")
        assert err <= 1e-2
