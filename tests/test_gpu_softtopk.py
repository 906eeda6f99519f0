"""GPU parity of sla_soft_topk against the oracle (SLA2 write-up §四: SoftTop-k,
a sigmoid with a temperature, threshold such that each row's weights sum to
k).  Both sides evaluate the pooled logits and the threshold in float64; the
GPU writes float32 weights, so the bar is float32 rounding: max-abs <= 2e-6
and every row summing to k within float32 accumulation."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, N, d, bq, bk, k_frac, T, router
    ("fp32-ragged-1000", "fp32", 1000, 64, 64, 64, 0.1, 0.5, False),
    ("bf16-ragged-1001-d128", "bf16", 1001, 128, 128, 64, 0.2, 0.05, False),
    ("bf16-router", "bf16", 2000, 128, 128, 64, 0.03, 1.0, True),
    ("bf16-bk128-cold", "bf16", 3000, 128, 128, 128, 0.25, 0.01, False),
    ("bf16-k0", "bf16", 700, 128, 128, 64, 0.0, 0.5, False),
    ("bf16-kall", "bf16", 700, 128, 128, 64, 1.0, 0.5, False),
]


def _check(x, k_frac, T):
    wl = x.wl
    q, k = U.dev(x.Q, x.K)
    wq, wk = U.dev(x.Wq, x.Wk)
    M = S.sla_soft_topk(q, k, wl.bq, wl.bk, k_frac, T, wq, wk)
    torch.cuda.synchronize()
    Mg = M.cpu().numpy().astype(np.float64)
    Mo = O.soft_topk(x.Q, x.K, wl.bq, wl.bk, k_frac, T, x.Wq, x.Wk)
    err = np.abs(Mg - Mo).max()
    Nk = Mo.shape[-1]
    kk = O.k_from_frac(k_frac, Nk)
    sums = Mg.sum(axis=-1)
    print(f"  max-abs {err:.3g}, row sums in [{sums.min():.6f}, {sums.max():.6f}] for k = {kk}")
    assert err <= 2e-6, f"max-abs {err}"
    assert np.all(np.abs(sums - kk) <= 1e-4 * max(1, kk)), (sums.min(), sums.max(), kk)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_soft_topk_small(case):
    name, dtype, N, d, bq, bk, k_frac, T, router = case
    print(f"[soft-topk] {name}", flush=True)
    wl = gen.Workload("adhoc", B=2, H=3, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=k_frac, p=0.0,
                      dtype=dtype, router=router, seed=9)
    _check(gen.make(wl), k_frac, T)


def test_soft_topk_480p_heads():
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print(f"[soft-topk] {wl.name}, 2 heads", flush=True)
    _check(gen.make(wl, heads=2), wl.k_frac, 0.5)
