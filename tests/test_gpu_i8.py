"""GPU parity of the 8-bit sparse branch (SLA2 write-up §三) against the
oracle.

* Codes and scales (sla_quantize_i8) are integer work decided by float32
  arithmetic that both sides perform identically: compared bit for bit.
* The output (sla_sparse_fwd_i8) is compared with the oracle's integer-exact
  definition on the same codes.  The one step the two sides cannot take
  identically is exp2 (the hardware instruction is within an ulp, the oracle
  rounds correctly), which can move a P code by one where 127 exp(S - m) lies
  within an ulp of a half-integer.  Each such flip moves an output by at most
  2 * 127 * sv_c / L (L = the query's sum of codes); the bound allows two
  flips per query, plus one unit in the last place of the output dtype.  The
  share of outputs off by more than that last-place unit is also bounded."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu


def _pos_to_key():
    """Key (within its 64-key tile) stored at byte pos of a V^T row."""
    k = np.zeros(64, dtype=np.int64)
    for pos in range(64):
        g, r = divmod(pos, 32)
        h, a, b = r // 16, (r % 16) // 4, r % 4
        k[pos] = 32 * g + 8 * a + 4 * h + b
    return k


def _codes_equal(x, qbuf, bq, bk, dtype):
    B, H, N, d = x.Q.shape
    v = S.i8_views(qbuf, (B, H, N, d), bq, bk, dtype)
    qz = O.quantize_i8(x.Q, x.K, x.V, bq, bk)
    BH = B * H
    q8 = v["q8"].cpu().numpy()
    k8 = v["k8"].cpu().numpy()
    np.testing.assert_array_equal(q8[:, :N], qz["q8"].reshape(BH, N, d))
    assert not q8[:, N:].any()
    np.testing.assert_array_equal(k8[:, :N], qz["k8"].reshape(BH, N, d))
    assert not k8[:, N:].any()
    vt = v["vt8"].cpu().numpy()                      # [BH, tiles, d, 64]
    ntile = vt.shape[1]
    v8 = np.zeros((BH, ntile * 64, d), dtype=np.int8)
    keys = _pos_to_key()
    for t in range(ntile):
        v8[:, t * 64 + keys, :] = vt[:, t].transpose(0, 2, 1)
    np.testing.assert_array_equal(v8[:, :N], qz["v8"].reshape(BH, N, d))
    assert not v8[:, N:].any()
    for name in ("sq", "sk", "sv"):
        np.testing.assert_array_equal(v[name].cpu().numpy(), qz[name].reshape(BH, -1), err_msg=name)
    return qz


def _out_check(og, qz, rp, ci, bq, bk, rows, dtype):
    """og: GPU output [B, H, N, d] on the host (float64)."""
    ref, sums = O.sparse_branch_i8(qz, bq, bk, rp, ci, rows=rows, with_sums=True)
    N = og.shape[2]
    ulp = 2.0 ** -7 if dtype == torch.bfloat16 else 2.0 ** -21
    worst, beyond, total = 0.0, 0, 0
    for (b, h, i), o in ref.items():
        s, e = O.block_range(i, bq, N)
        g = og[b, h, s:e]
        L = sums[(b, h, i)].astype(np.float64)
        sv = qz["sv"][b, h].astype(np.float64)
        flip = np.where(L[:, None] > 0, 2 * 2 * 127 * sv[None, :] / np.maximum(L[:, None], 1), 0.0)
        tol = ulp * np.abs(o) + flip + 1e-30
        err = np.abs(g - o)
        assert np.all(err <= tol), (b, h, i, float((err - tol).max()))
        worst = max(worst, float((err / tol).max()))
        beyond += int((err > ulp * np.abs(o) + 1e-30).sum())
        total += err.size
    print(f"  worst err/tol {worst:.3g}; beyond one ulp {beyond} of {total}")
    assert beyond <= max(2, total // 200)


def _random_csr(rng, R, Nk, density, empty_rows=(), full_rows=()):
    rp, ci = [0], []
    for r in range(R):
        if r in empty_rows:
            sel = np.zeros(0, dtype=np.int64)
        elif r in full_rows:
            sel = np.arange(Nk)
        else:
            sel = np.flatnonzero(rng.random(Nk) < density)
        ci.extend(sel.tolist())
        rp.append(len(ci))
    return np.array(rp, dtype=np.int64), np.array(ci, dtype=np.int64)


CASES = [
    # name, dtype, N, d, bq, bk, density
    ("bf16-ragged-1000", "bf16", 1000, 128, 128, 64, 0.3),
    ("fp32-d64-bk128-777", "fp32", 777, 64, 64, 128, 0.4),
    ("bf16-bq64-bk128-1500", "bf16", 1500, 128, 64, 128, 0.25),
    ("bf16-d64-600", "bf16", 600, 64, 128, 64, 0.5),
    ("fp32-d128-bq64-300", "fp32", 300, 128, 64, 64, 0.6),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_i8_small(case):
    name, dt, N, d, bq, bk, density = case
    print(f"[i8] {name}", flush=True)
    wl = gen.Workload("adhoc", B=1, H=3, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype=dt, router=False, seed=11)
    x = gen.make(wl)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q, k, v = U.dev(x.Q, x.K, x.V)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rng = np.random.default_rng(5)
    rp, ci = _random_csr(rng, 3 * Nq, Nk, density, empty_rows={1}, full_rows={2, 3 * Nq - 1})
    qbuf = S.sla_quantize_i8(q, k, v, bq, bk)
    og = S.sla_sparse_fwd_i8(qbuf, q, bq, bk, torch.from_numpy(rp).int().cuda(),
                             torch.from_numpy(ci).int().cuda() if len(ci) else torch.zeros(1, dtype=torch.int32,
                                                                                           device="cuda"))
    torch.cuda.synchronize()
    qz = _codes_equal(x, qbuf, bq, bk, tdt)
    _out_check(og.cpu().double().numpy(), qz, rp, ci, bq, bk, None, tdt)


def test_i8_degenerate_scales():
    """A query block of zeros (sq = 0: every listed key scores 0, all codes
    127, a plain mean), a V channel of zeros (sv = 0) and a V channel with one
    non-zero value."""
    print("[i8] degenerate scales", flush=True)
    N, d, bq, bk = 500, 128, 128, 64
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.0,
                      dtype="bf16", router=False, seed=12)
    x = gen.make(wl)
    x.Q[0, 0, 128:256] = 0
    x.V[0, 1, :, 5] = 0
    x.V[0, 1, :, 7] = 0
    x.V[0, 1, 300, 7] = 3.0
    q, k, v = U.dev(x.Q, x.K, x.V)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = _random_csr(np.random.default_rng(6), 2 * Nq, Nk, 0.5, full_rows={1})
    qbuf = S.sla_quantize_i8(q, k, v, bq, bk)
    og = S.sla_sparse_fwd_i8(qbuf, q, bq, bk, torch.from_numpy(rp).int().cuda(), torch.from_numpy(ci).int().cuda())
    torch.cuda.synchronize()
    qz = _codes_equal(x, qbuf, bq, bk, torch.bfloat16)
    assert qz["sq"][0, 0, 1] == 0 and qz["sv"][0, 1, 5] == 0
    o = og.cpu().double().numpy()
    assert not o[0, 1, :, 5].any()
    _out_check(o, qz, rp, ci, bq, bk, None, torch.bfloat16)


def test_i8_480p_sampled_rows():
    """The 480p SLA2 workload (N = 32760, d = 128, bq 128, bk 64) at full
    length on two heads, with the library's own mask: codes bit for bit, and
    the output on sampled rows of both heads."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[i8] {wl.name}, 2 heads", flush=True)
    x = gen.make(wl, heads=2)
    q, k, v = U.dev(x.Q, x.K, x.V)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    qbuf = S.sla_quantize_i8(q, k, v, wl.bq, wl.bk)
    og = S.sla_sparse_fwd_i8(qbuf, q, wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    rp, ci = U.csr(rp_t, ci_t)
    qz = _codes_equal(x, qbuf, wl.bq, wl.bk, torch.bfloat16)
    Nq = O.n_blocks(wl.N, wl.bq)
    rng = np.random.default_rng(7)
    rows = [(0, h, int(i)) for h in range(2) for i in rng.choice(Nq, 6, replace=False)] + [(0, 1, Nq - 1)]
    _out_check(og.cpu().double().numpy(), qz, rp, ci, wl.bq, wl.bk, rows, torch.bfloat16)
