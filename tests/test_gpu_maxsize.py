"""The longest mask rows the library accepts: Nk = 4096 key blocks per row
(N = 262144 tokens at bk = 64), the limit of the selection's lane x slot
layout, with an exact and a ragged last block, on a peaked map (Top-k
decides, short rows) and a flat one (Top-p keeps a large part of each row).
The mask is compared with the oracle's as in the other mask tests; the fused
forward on sampled row blocks (the longest and shortest rows, the last one)
with the bf16 bar; and the mixed backward there (dQ of sampled row blocks
against the oracle, dV summed over the keys against dO summed over the
queries)."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U
from tests.test_gpu_bwd import _compare

pytestmark = pytest.mark.gpu

NK_MAX = 4096
CASES = [
    # name, N, tau, k_frac, p
    ("peaked-exact", NK_MAX * 64, 1.0, 0.02, 0.7),
    ("peaked-ragged", NK_MAX * 64 - 17, 1.0, 0.02, 0.7),
    ("flat-ragged", NK_MAX * 64 - 17, 0.25, 0.01, 0.9),
]


def _inputs(N, tau, k_frac, p):
    wl = gen.Workload("adhoc", B=1, H=1, grid=(1, 1, N), d=64, bq=128, bk=64, k_frac=k_frac, p=p,
                      dtype="bf16", router=False, seed=37, tau=tau, alpha=(0.7,))
    return gen.make(wl)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mask_at_the_longest_rows(case):
    name, N, tau, k_frac, p = case
    print(f"[maxsize] mask {name}: N {N}", flush=True)
    x = _inputs(N, tau, k_frac, p)
    wl = x.wl
    assert O.n_blocks(N, wl.bk) == NK_MAX
    q, k = U.dev(x.Q, x.K)
    rp, ci, logits = S.sla_mask(q, k, wl.bq, wl.bk, k_frac, p, return_logits=True)
    torch.cuda.synchronize()
    rp_g, ci_g = U.csr(rp, ci)
    rp_o, ci_o, meta = U.oracle_mask_per_head(x, k_frac, p)
    Nq = O.n_blocks(N, wl.bq)
    U.check_csr_structure(rp_g, ci_g, Nq, NK_MAX)
    Sg = logits.cpu().numpy().reshape(meta["S"].shape)
    err = np.max(np.abs(Sg - meta["S"]) / np.maximum(1.0, np.abs(meta["S"])))
    assert err < 1e-10, f"pooled logits differ by {err}"
    bad, excused, rows = U.mask_mismatches(rp_g, ci_g, rp_o, ci_o, meta, p)
    counts = np.diff(rp_g)
    print(f"  blocks per row {counts.min()}..{counts.max()}, differing rows {rows}, excused {excused}")
    assert not bad, f"{len(bad)} unexcused mask differences, e.g. {bad[:5]}"
    assert counts.min() >= meta["k"]


def test_fused_forward_at_the_longest_rows():
    name, N, tau, k_frac, p = CASES[2]
    print(f"[maxsize] fused forward {name}: N {N}", flush=True)
    x = _inputs(N, tau, k_frac, p)
    wl = x.wl
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    o, rp, ci = S.sla_attn_fwd(q, k, v, a, wl.bq, wl.bk, k_frac, p)
    torch.cuda.synchronize()
    rp_g, ci_g = U.csr(rp, ci)
    counts = np.diff(rp_g)
    Nq = len(counts)
    rows = sorted({(0, 0, int(np.argmax(counts))), (0, 0, int(np.argmin(counts))), (0, 0, Nq // 3),
                   (0, 0, Nq - 1)})
    print(f"  blocks per row {counts.min()}..{counts.max()}, rows {[r[2] for r in rows]}", flush=True)
    ref_s = O.sparse_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp_g, ci_g, rows)
    ref_l = O.linear_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp_g, ci_g, rows)
    ref = {r: O.combine(ref_s[r], ref_l[r], 0.7) for r in rows}
    m, rel = U.compare_rows(U.rows_of(o, rows, wl.bq), ref)
    print(f"  o: max-abs {m:.3g} rel {rel:.3g}")
    assert m <= 2e-2 and rel <= 5e-3


def test_mixed_backward_at_the_longest_rows():
    name, N, tau, k_frac, p = CASES[2]
    print(f"[maxsize] sla_attn_bwd {name}: N {N}", flush=True)
    x = _inputs(N, tau, k_frac, p)
    wl = x.wl
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    rp_t, ci_t = S.sla_mask(q, k, wl.bq, wl.bk, k_frac, p)
    rp, ci = U.csr(rp_t, ci_t)
    counts = np.diff(rp)
    assert counts.min() > 0 and counts.max() < NK_MAX  # both branches on every row
    dO = torch.from_numpy(np.random.default_rng(17).normal(size=tuple(x.Q.shape))).to(torch.bfloat16)
    dq, dk, dv = S.sla_attn_bwd(q, k, v, dO.cuda(), a, wl.bq, wl.bk, rp_t, ci_t)
    torch.cuda.synchronize()
    Nq = len(counts)
    rows = sorted({(0, 0, int(np.argmax(counts))), (0, 0, int(np.argmin(counts))), (0, 0, Nq - 1)})
    rs = O.sparse_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    rl = O.linear_branch_backward(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, dO, rows=rows)
    for (b, h, i) in rows:
        s, e = O.block_range(i, wl.bq, N)
        ref = 0.7 * rs["dQ"][b, h, s:e] + 0.3 * rl["dQ"][b, h, s:e]
        _compare(dq[b, h, s:e], ref, f"dQ rows of block {i}")
    G = O.as_f64(dO)[0, 0]
    err = np.abs(dv[0, 0].cpu().double().numpy().sum(0) - G.sum(0)).max() / np.abs(G).sum(0).max()
    print(f"  sum dV vs sum dO: {err:.3g} of sum|dO|")
    assert err <= 1e-2
