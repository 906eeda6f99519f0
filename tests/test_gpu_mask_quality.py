"""The mask-quality study's figures (mask_quality.py: kept fraction, pooled
mass, token-level mass of each selection rule; SpargeAttention2 write-up §一
and §六 on flat versus peaked maps) checked against the oracle on the same
inputs: two heads of the routed 480p workload at a flat (tau = 0.25) and a
peaked (tau = 4) temperature, p = 0.6, for Top-k alone, Top-p alone and the
union."""
import math

import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
import mask_quality as MQ
from oracle import sla_oracle as O

pytestmark = pytest.mark.gpu


def _token_mass_f64(Q, K, bq, bk, rp, ci, samples):
    """Exact softmax mass on the selected keys, float64 on the CPU, averaged
    over the queries of each sampled block and then over the blocks."""
    Qd, Kd = O.as_f64(Q), O.as_f64(K)
    N, d = Qd.shape[2], Qd.shape[3]
    Nq = O.n_blocks(N, bq)
    tot = 0.0
    for (h, i) in samples:
        r = h * Nq + i
        keys = np.concatenate([np.arange(*O.block_range(int(j), bk, N)) for j in ci[rp[r]:rp[r + 1]]]
                              or [np.zeros(0, np.int64)])
        s, e = O.block_range(i, bq, N)
        A = Qd[0, h, s:e] @ Kd[0, h].T / math.sqrt(d)
        A = np.exp(A - A.max(axis=1, keepdims=True))
        A /= A.sum(axis=1, keepdims=True)
        tot += A[:, keys].sum(axis=1).mean()
    return tot / len(samples)


@pytest.mark.parametrize("tau", [0.25, 4.0])
def test_study_figures_match_the_oracle(tau):
    wl = gen.WORKLOADS["video480p-router-N32760"].with_(tau=tau)
    print(f"[mask-quality] tau={tau}", flush=True)
    x = gen.make(wl, heads=2)
    q, k = (t.cuda().contiguous() for t in (x.Q, x.K))
    wq, wk = x.Wq.cuda(), x.Wk.cuda()
    rng = np.random.default_rng(4)
    samples = [(h, int(i)) for h in range(2) for i in rng.choice(wl.Nq, 2, replace=False)]
    p = 0.6
    for rule, kf, pp in (("topk", wl.k_frac, 0.0), ("topp", 0.0, p), ("union", wl.k_frac, p)):
        rp, ci, st = MQ.rule_stats(S, q, k, wl, wq, wk, kf, pp, samples)
        rp_o, ci_o, meta = O.mask(x.Q, x.K, wl.bq, wl.bk, kf, pp, x.Wq, x.Wk, keep_info=False)
        R = 2 * wl.Nq
        kept = len(ci_o) / float(R * wl.Nk)
        P = meta["P"].reshape(R, wl.Nk)
        pooled = np.mean([P[r, ci_o[rp_o[r]:rp_o[r + 1]]].sum() for r in range(R)])
        token = _token_mass_f64(x.Q, x.K, wl.bq, wl.bk, rp_o, ci_o, samples)
        print(f"  {rule}: kept {st['kept']:.4f}/{kept:.4f} pooled {st['pooled_mass']:.6f}/{pooled:.6f} "
              f"token {st['token_mass']:.5f}/{token:.5f}")
        assert st["kept"] == kept
        assert abs(st["pooled_mass"] - pooled) <= 1e-9
        assert abs(st["token_mass"] - token) <= 1e-4
