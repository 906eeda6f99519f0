"""Pins of the oracle's SoftTop-k (SLA2 write-up §四: a sigmoid with a
temperature replaces the hard Top-k in the router's first training stage).

The reading: M_j = sigmoid((S_j - tau) / T) with tau such that sum_j M_j = k.
Pinned here by closed forms and by the properties that fix it: two blocks
(tau is the midpoint), all-equal logits (every weight k / Nk), the weights
summing to k, the hard Top-k limit as T -> 0, invariance under a common shift,
strict monotonicity, and the k = 0 / k = Nk edges."""
import math

import numpy as np
import pytest

from oracle import sla_oracle as O


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


@pytest.mark.parametrize("a,b,T", [(1.0, 3.0, 0.5), (-2.0, 5.0, 1.5), (0.25, 0.2, 0.01)])
def test_two_blocks_closed_form(a, b, T):
    M, tau = O.soft_topk_row(np.array([a, b]), 1, T)
    assert tau == pytest.approx(0.5 * (a + b), abs=1e-12)
    assert M[0] == pytest.approx(_sig((a - b) / (2 * T)), abs=1e-14)
    assert M[1] == pytest.approx(_sig((b - a) / (2 * T)), abs=1e-14)


@pytest.mark.parametrize("k,Nk", [(1, 7), (3, 16), (16, 512)])
def test_equal_logits_share_k_evenly(k, Nk):
    M, tau = O.soft_topk_row(np.full(Nk, 2.5), k, 0.3)
    np.testing.assert_allclose(M, np.full(Nk, k / Nk), atol=1e-13)
    # sigmoid((2.5 - tau) / T) = k / Nk
    assert tau == pytest.approx(2.5 - 0.3 * math.log((k / Nk) / (1 - k / Nk)), abs=1e-12)


@pytest.mark.parametrize("seed,k,T", [(0, 16, 0.1), (1, 26, 1.0), (2, 3, 0.02), (3, 100, 5.0)])
def test_weights_sum_to_k_and_are_monotone(seed, k, T):
    S = np.random.default_rng(seed).normal(size=512) * 4.0
    M, _ = O.soft_topk_row(S, k, T)
    assert M.sum() == pytest.approx(k, abs=1e-9)
    assert np.all((M >= 0) & (M <= 1))
    order = np.argsort(S)
    assert np.all(np.diff(M[order]) >= 0)


def test_small_temperature_gives_hard_topk():
    rng = np.random.default_rng(4)
    S = np.sort(rng.choice(np.arange(1000), size=64, replace=False)).astype(np.float64)  # gaps >= 1
    rng.shuffle(S)
    k = 10
    M, _ = O.soft_topk_row(S, k, 0.01)
    hard = np.zeros(64)
    hard[np.argsort(-S)[:k]] = 1.0
    np.testing.assert_allclose(M, hard, atol=1e-12)


def test_common_shift_moves_only_the_threshold():
    S = np.random.default_rng(5).normal(size=100)
    M1, t1 = O.soft_topk_row(S, 7, 0.4)
    M2, t2 = O.soft_topk_row(S + 123.0, 7, 0.4)
    np.testing.assert_allclose(M1, M2, atol=1e-12)
    assert t2 - t1 == pytest.approx(123.0, abs=1e-9)


def test_edges():
    S = np.random.default_rng(6).normal(size=9)
    M0, t0 = O.soft_topk_row(S, 0, 1.0)
    M9, t9 = O.soft_topk_row(S, 9, 1.0)
    assert np.all(M0 == 0) and t0 == math.inf
    assert np.all(M9 == 1) and t9 == -math.inf


def test_mask_shape_and_counts():
    import gen
    wl = gen.Workload("adhoc", B=1, H=2, grid=(1, 1, 700), d=64, bq=64, bk=64, k_frac=0.25, p=0.0,
                      dtype="fp32", router=False, seed=3)
    x = gen.make(wl)
    M = O.soft_topk(x.Q, x.K, wl.bq, wl.bk, wl.k_frac, 0.5)
    Nq, Nk = O.n_blocks(700, 64), O.n_blocks(700, 64)
    assert M.shape == (1, 2, Nq, Nk)
    np.testing.assert_allclose(M.sum(axis=-1), O.k_from_frac(wl.k_frac, Nk), atol=1e-9)
