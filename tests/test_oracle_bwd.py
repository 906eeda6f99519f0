"""Pins of the oracle's sparse-branch backward and alpha gradient: central
finite differences of the forward definition on a tiny ragged case (every
input element), the full-mask case against dense attention's gradient through
torch's scaled_dot_product_attention in float64, rows with no selected block,
and the alpha gradient against a finite difference of the mixed output."""
import numpy as np
import pytest
import torch

from oracle import sla_oracle as O


def _tiny(seed=0, N=11, d=4, bq=4, bk=3):
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.normal(size=(1, 2, N, d)) for _ in range(4))
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = [0], []
    for r in range(2 * Nq):
        sel = [j for j in range(Nk) if rng.random() < 0.5] if r != 1 else []
        ci.extend(sel)
        rp.append(len(ci))
    return Q, K, V, dO, np.array(rp), np.array(ci, dtype=np.int64), bq, bk


def _loss(Q, K, V, dO, rp, ci, bq, bk):
    out = O.sparse_branch(Q, K, V, bq, bk, rp, ci)
    N = Q.shape[2]
    return sum(float((o * dO[b, h, slice(*O.block_range(i, bq, N))]).sum()) for (b, h, i), o in out.items())


def test_finite_differences_every_element():
    Q, K, V, dO, rp, ci, bq, bk = _tiny()
    g = O.sparse_branch_backward(Q, K, V, bq, bk, rp, ci, dO)
    eps = 1e-6
    for name, X in (("dQ", Q), ("dK", K), ("dV", V)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args = {"dQ": (Xp, K, V), "dK": (Q, Xp, V), "dV": (Q, K, Xp)}[name]
            argm = {"dQ": (Xm, K, V), "dK": (Q, Xm, V), "dV": (Q, K, Xm)}[name]
            num[idx] = (_loss(*args, dO, rp, ci, bq, bk) - _loss(*argm, dO, rp, ci, bq, bk)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_empty_row_contributes_nothing():
    Q, K, V, dO, rp, ci, bq, bk = _tiny(seed=1)
    g = O.sparse_branch_backward(Q, K, V, bq, bk, rp, ci, dO)
    # row r = 1 is (b 0, h 0, query block 1) and selects nothing
    assert not g["dQ"][0, 0, 4:8].any()
    dO2 = dO.copy()
    dO2[0, 0, 4:8] = 123.0    # its upstream gradient has no effect anywhere
    g2 = O.sparse_branch_backward(Q, K, V, bq, bk, rp, ci, dO2)
    for k in g:
        np.testing.assert_array_equal(g[k], g2[k])


def test_full_mask_is_dense_gradient():
    rng = np.random.default_rng(2)
    N, d, bq, bk = 37, 8, 8, 16
    Q, K, V, dO = (rng.normal(size=(1, 2, N, d)) for _ in range(4))
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp = np.arange(0, 2 * Nq + 1) * Nk
    ci = np.tile(np.arange(Nk), 2 * Nq)
    g = O.sparse_branch_backward(Q, K, V, bq, bk, rp, ci, dO)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    torch.nn.functional.scaled_dot_product_attention(q, k, v).backward(torch.tensor(dO))
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), atol=1e-12, err_msg=name)


def test_alpha_gradient_finite_difference():
    Q, K, V, dO, rp, ci, bq, bk = _tiny(seed=3)
    Os = O.assemble(O.sparse_branch(Q, K, V, bq, bk, rp, ci), 1, 2, 11, 4, bq)
    Ol = O.assemble(O.linear_branch(Q, K, V, bq, bk, rp, ci), 1, 2, 11, 4, bq)
    ga = O.alpha_grad(dO, Os, Ol)
    for h in range(2):
        def loss(a):
            return float((dO[:, h] * O.combine(Os[:, h], Ol[:, h], a)).sum())
        num = (loss(0.3 + 1e-6) - loss(0.3 - 1e-6)) / 2e-6
        assert ga[h] == pytest.approx(num, abs=1e-7)


def _loss_lin(Q, K, V, dO, rp, ci, bq, bk):
    out = O.linear_branch(Q, K, V, bq, bk, rp, ci)
    N = Q.shape[2]
    return sum(float((o * dO[b, h, slice(*O.block_range(i, bq, N))]).sum()) for (b, h, i), o in out.items())


def test_linear_finite_differences_every_element():
    Q, K, V, dO, rp, ci, bq, bk = _tiny(seed=10)
    g = O.linear_branch_backward(Q, K, V, bq, bk, rp, ci, dO)
    eps = 1e-6
    for name, X in (("dQ", Q), ("dK", K), ("dV", V)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args = {"dQ": (Xp, K, V), "dK": (Q, Xp, V), "dV": (Q, K, Xp)}[name]
            argm = {"dQ": (Xm, K, V), "dK": (Q, Xm, V), "dV": (Q, K, Xm)}[name]
            num[idx] = (_loss_lin(*args, dO, rp, ci, bq, bk) - _loss_lin(*argm, dO, rp, ci, bq, bk)) / (2 * eps)
        np.testing.assert_allclose(g[name], num, atol=1e-7, rtol=1e-6, err_msg=name)


def test_linear_gradient_invariants():
    """Weights over the unselected keys sum to one, so sum_u dV_u = sum of dO
    over the rows with any unselected key; O_l is unchanged by scaling
    phi(q_t), so sum_r (dq_t[r] / phi'(q_t[r])) phi(q_t[r]) = 0; a row whose
    blocks are all selected contributes nothing."""
    Q, K, V, dO, rp, ci, bq, bk = _tiny(seed=11, N=13)
    Nq, Nk = O.n_blocks(13, bq), O.n_blocks(13, bk)
    rp = list(rp)
    ci = list(ci)
    # make row 0 (b 0, h 0, block 0) select every block
    n0 = rp[1] - rp[0]
    ci = list(range(Nk)) + ci[n0:]
    rp = [0] + [x - n0 + Nk for x in rp[1:]]
    rp, ci = np.array(rp), np.array(ci, dtype=np.int64)
    g = O.linear_branch_backward(Q, K, V, bq, bk, rp, ci, dO)
    assert not g["dQ"][0, 0, 0:4].any()
    for h in range(2):
        rows_with = np.zeros(13, dtype=bool)
        for i in range(Nq):
            r = h * Nq + i
            if rp[r + 1] - rp[r] < Nk:
                rows_with[slice(*O.block_range(i, bq, 13))] = True
        np.testing.assert_allclose(g["dV"][0, h].sum(axis=0), dO[0, h][rows_with].sum(axis=0), atol=1e-12)
    phi = np.where(Q > 0, Q + 1.0, np.exp(np.minimum(Q, 0.0)))
    dphi = np.where(Q > 0, 1.0, np.exp(np.minimum(Q, 0.0)))
    np.testing.assert_allclose(((g["dQ"] / dphi) * phi).sum(axis=-1), 0.0, atol=1e-12)
