"""GPU parity of the sparse-branch backward and the alpha gradient against
the oracle (float64 autograd of the forward definition, mask fixed).

Bar, derived from the arithmetic: the kernels take bf16 inputs exactly,
recompute S in float32 (D too, as sum_u P dP), and round two things to bf16 -
P and dS where they enter a matrix product (relative 2^-9 each) - and the
outputs (2^-9).  Those roundings are independent from element to
element, so each gradient tensor must stay within a relative L1 error of
1e-2 of the exact one, and every element within 2e-2 of the tensor's largest
magnitude.  Key blocks that no row lists get exactly zero dK and dV; the
alpha gradient (float64 sums, float32 result) matches to 1e-5 relative."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu


def _random_csr(rng, BH, Nq, Nk, density, empty_rows=(), full_rows=(), unused_col=None):
    rp, ci = [0], []
    for r in range(BH * Nq):
        if r in empty_rows:
            sel = np.zeros(0, dtype=np.int64)
        elif r in full_rows:
            sel = np.arange(Nk)
        else:
            sel = np.flatnonzero(rng.random(Nk) < density)
        if unused_col is not None:
            sel = sel[sel != unused_col]
        ci.extend(sel.tolist())
        rp.append(len(ci))
    return np.array(rp, dtype=np.int64), np.array(ci, dtype=np.int64)


def _compare(got, ref, name):
    g = got.cpu().double().numpy()
    rel = np.abs(g - ref).sum() / max(np.abs(ref).sum(), 1e-30)
    mx = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30)
    print(f"  {name}: rel-L1 {rel:.3g}, max-abs/max|ref| {mx:.3g}")
    assert rel <= 1e-2 and mx <= 2e-2, (name, rel, mx)


def _run(x, bq, bk, rp, ci, seed):
    q, k, v = U.dev(x.Q, x.K, x.V)
    dO = torch.from_numpy(np.random.default_rng(seed).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    g = dO.cuda()
    rpt = torch.from_numpy(rp).int().cuda()
    cit = torch.from_numpy(ci).int().cuda() if len(ci) else torch.zeros(1, dtype=torch.int32, device="cuda")
    dq, dk, dv = S.sla_sparse_bwd(q, k, v, g, bq, bk, rpt, cit)
    torch.cuda.synchronize()
    ref = O.sparse_branch_backward(x.Q, x.K, x.V, bq, bk, rp, ci, dO)
    _compare(dq, ref["dQ"], "dQ")
    _compare(dk, ref["dK"], "dK")
    _compare(dv, ref["dV"], "dV")
    return dq, dk, dv


CASES = [
    # name, N, d, bq, bk, density
    ("ragged-1000", 1000, 128, 128, 64, 0.3),
    ("d64-bq64-bk128-777", 777, 64, 64, 128, 0.4),
    ("bq64-bk128-1500", 1500, 128, 64, 128, 0.25),
    ("d64-600", 600, 64, 128, 64, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sparse_bwd_small(case):
    name, N, d, bq, bk, density = case
    print(f"[bwd] {name}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=21)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(8), 2, Nq, Nk, density, empty_rows={1},
                         full_rows={2 * Nq - 1}, unused_col=2)
    dq, dk, dv = _run(x, bq, bk, rp, ci, seed=4)
    # key block 2 is listed by no row of either head
    assert not dk[0, :, 2 * bk:3 * bk].any() and not dv[0, :, 2 * bk:3 * bk].any()


def _skewed_csr(rng, BH, Nq, Nk):
    """Columns listed with very different frequencies, so that the column
    kernels' launch order (most-listed key blocks first) spans its classes:
    block 0 and the last (ragged) block by every row, block 1 by every second
    row, block 3 by no row, the rest at random by about 10% of the rows."""
    rp, ci = [0], []
    for r in range(BH * Nq):
        sel = set(np.flatnonzero(rng.random(Nk) < 0.1).tolist()) | {0, Nk - 1}
        if r % 2 == 0:
            sel.add(1)
        sel.discard(3)
        ci.extend(sorted(sel))
        rp.append(len(ci))
    return np.array(rp, dtype=np.int64), np.array(ci, dtype=np.int64)


@pytest.mark.parametrize("bk", [64, 128])
def test_sparse_bwd_skewed_columns(bk):
    N, d, bq = 4000, 128, 128
    print(f"[bwd] skewed columns bk={bk}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=31)
    x = gen.make(wl)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _skewed_csr(np.random.default_rng(13), 2, Nq, Nk)
    dq, dk, dv = _run(x, bq, bk, rp, ci, seed=9)
    assert not dk[0, :, 3 * bk:4 * bk].any() and not dv[0, :, 3 * bk:4 * bk].any()


def test_sparse_bwd_480p_two_heads():
    """The 480p SLA2 workload at full length (N = 32760) on two heads with the
    library's own mask."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[bwd] {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k = U.dev(x.Q, x.K)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    _run(x, wl.bq, wl.bk, rp, ci, seed=5)


def test_sparse_bwd_720p_one_head():
    """The 720p SLA2 workload at full length (N = 75600, 591 x 1182 blocks) on
    one head with the library's mask.  The oracle differentiates sampled row
    blocks (the longest and shortest rows, the middle one and the ragged last
    one: their dQ rows are exact); every key is checked by two identities
    that hold at any size: sum_u dV_u = sum_t dO_t over the rows with a
    listed block (P's rows sum to 1), and sum_u dK_u = 0 (each row's dS sums
    to 0, sum_u P_tu (dP_tu - D_t) = D_t - D_t)."""
    wl = gen.WORKLOADS["video720p-sla2-N75600"]
    print(f"[bwd] {wl.name}, 1 head", flush=True)
    x = gen.make(wl, heads=1)
    q, k, v = U.dev(x.Q, x.K, x.V)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    rp, ci = U.csr(rp_t, ci_t)
    dO = torch.from_numpy(np.random.default_rng(15).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    dq, dk, dv = S.sla_sparse_bwd(q, k, v, dO.cuda(), wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    N = x.Q.shape[2]
    counts = np.diff(rp)
    Nq = len(counts)
    rows = sorted({(0, 0, int(np.argmax(counts))), (0, 0, int(np.argmin(counts))), (0, 0, 137),
                   (0, 0, Nq // 2), (0, 0, Nq - 1)})
    print(f"  blocks per row {counts.min()}..{counts.max()}, sampled rows {[r[2] for r in rows]}")
    ref = O.sparse_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    for (b, h, i) in rows:
        s, e = O.block_range(i, wl.bq, N)
        _compare(dq[b, h, s:e], ref["dQ"][b, h, s:e], f"dQ rows of block {i}")
    G = O.as_f64(dO)[0, 0]
    dkd, dvd = dk[0, 0].cpu().double().numpy(), dv[0, 0].cpu().double().numpy()
    has = np.repeat(counts > 0, wl.bq)[:N]
    err = np.abs(dvd.sum(0) - G[has].sum(0)).max() / np.abs(G[has]).sum(0).max()
    print(f"  sum dV vs sum dO: {err:.3g} of sum|dO|")
    assert err <= 1e-2
    rel = (np.abs(dkd.sum(0)) / np.maximum(np.abs(dkd).sum(0), 1e-30)).max()
    print(f"  sum dK: {rel:.3g} of sum|dK| (worst column)")
    assert rel <= 1e-2


def test_alpha_grad():
    print("[bwd] alpha gradient", flush=True)
    rng = np.random.default_rng(9)
    shape = (2, 3, 1000, 64)
    dO, Os, Ol = (torch.from_numpy(rng.normal(size=shape)).to(torch.bfloat16) for _ in range(3))
    ga = S.sla_alpha_grad(dO.cuda(), Os.cuda(), Ol.cuda()).cpu().double().numpy()
    ref = O.alpha_grad(dO, Os, Ol)
    np.testing.assert_allclose(ga, ref, rtol=1e-5, atol=1e-6)
    f32 = [t.float() for t in (dO, Os, Ol)]
    gf = S.sla_alpha_grad(*(t.cuda() for t in f32)).cpu().double().numpy()
    np.testing.assert_allclose(gf, O.alpha_grad(*f32), rtol=1e-5, atol=1e-6)
