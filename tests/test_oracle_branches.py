"""Pins of the oracle's pooling, branches and combine against special cases
that reduce to independent library routines (torch fp64 on the CPU), closed
forms and brute-force token loops (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gen
from oracle import sla_oracle as O


def _qkv(B, H, N, d, seed, scale=1.0):
    q, k, v = gen.random_qkv(B, H, N, d, "fp32", seed, scale=scale)
    return q.double(), k.double(), v.double()


def _full(blocks, B, H, N, d, bq):
    return O.assemble(blocks, B, H, N, d, bq)


def _sdpa(q, k, v, mask=None):
    """torch's own attention routine, fp64 on the CPU."""
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask)


def _elu1(x):
    return F.elu(x) + 1.0


def test_phi_is_elu_plus_one():
    x = torch.linspace(-30, 30, 4001, dtype=torch.float64)
    assert np.array_equal(O.phi(x.numpy()), _elu1(x).numpy()) or \
        np.max(np.abs(O.phi(x.numpy()) - _elu1(x).numpy())) < 1e-15


@pytest.mark.parametrize("N,bq,bk", [(256, 64, 64), (200, 64, 32), (1000, 64, 64), (1001, 128, 64)])
def test_full_mask_alpha1_is_dense_attention(N, bq, bk):
    """alpha = 1 with every block selected (k_frac = 1) is plain dense softmax
    attention softmax(QK^T/sqrt(d))V."""
    B, H, d = 1, 2, 16
    q, k, v = _qkv(B, H, N, d, seed=N)
    rp, ci, meta = O.mask(q, k, bq, bk, 1.0, 0.5)
    assert len(ci) == B * H * meta["Nq"] * meta["Nk"]
    out = _full(O.attn(q, k, v, np.ones(H), bq, bk, rp, ci), B, H, N, d, bq)
    ref = _sdpa(q, k, v).numpy()
    assert np.max(np.abs(out - ref)) < 1e-12
    # the oracle's own dense routine agrees with torch too
    dn = _full(O.dense(q, k, v, bq=bq), B, H, N, d, bq)
    assert np.max(np.abs(dn - ref)) < 1e-12


@pytest.mark.parametrize("N,bq,bk", [(256, 64, 64), (333, 64, 32)])
def test_empty_mask_alpha0_is_linear_attention(N, bq, bk):
    """alpha = 0 with no block selected (k_frac = 0, p = 0) is textbook linear
    attention phi(Q)(phi(K)^T V) / phi(Q)(phi(K)^T 1), computed here by the
    associative (d x d summary) route with torch's elu."""
    B, H, d = 1, 2, 16
    q, k, v = _qkv(B, H, N, d, seed=7 + N, scale=0.5)
    rp, ci, meta = O.mask(q, k, bq, bk, 0.0, 0.0)
    assert len(ci) == 0
    out = _full(O.attn(q, k, v, np.zeros(H), bq, bk, rp, ci), B, H, N, d, bq)
    fq, fk = _elu1(q), _elu1(k)
    kv = fk.transpose(-1, -2) @ v                 # [B,H,d,d]
    z = fk.sum(dim=-2, keepdim=True)              # [B,H,1,d]
    ref = (fq @ kv) / (fq * z).sum(-1, keepdim=True)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def _token_mask(rp, ci, B, H, N, bq, bk):
    """Token-level boolean mask M[b,h,t,u] = block(u) selected by block(t)."""
    Nq = O.n_blocks(N, bq)
    M = torch.zeros((B, H, N, N), dtype=torch.bool)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                r = (b * H + h) * Nq + i
                s, e = O.block_range(i, bq, N)
                for j in ci[rp[r]:rp[r + 1]]:
                    ks, ke = O.block_range(int(j), bk, N)
                    M[b, h, s:e, ks:ke] = True
    return M


@pytest.mark.parametrize("N,bq,bk", [(1000, 64, 64), (1001, 64, 64), (777, 128, 64)])
def test_branches_against_token_mask_formulation(N, bq, bk):
    """With a partial mask and ragged last blocks, the sparse branch equals
    torch attention under the token-level boolean mask, and the linear branch
    equals the masked direct sum over the complement."""
    B, H, d = 1, 2, 16
    q, k, v = _qkv(B, H, N, d, seed=3 * N)
    rp, ci, meta = O.mask(q, k, bq, bk, 0.1, 0.4)
    M = _token_mask(rp, ci, B, H, N, bq, bk)
    assert 0 < int(M.sum()) < B * H * N * N
    Os = _full(O.sparse_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    ref_s = _sdpa(q, k, v, M).numpy()
    assert np.max(np.abs(Os - ref_s)) < 1e-12
    Ol = _full(O.linear_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    A = (_elu1(q) @ _elu1(k).transpose(-1, -2)) * (~M)
    ref_l = (A @ v) / A.sum(-1, keepdim=True)
    assert np.max(np.abs(Ol - ref_l.numpy())) < 1e-12


def test_decomposition_identity():
    """dense = beta * O_sparse + (1 - beta) * O_rest, beta = softmax mass of the
    selected keys: pins the renormalisation of the sparse branch."""
    B, H, N, d, bq, bk = 1, 2, 512, 32, 64, 64
    q, k, v = _qkv(B, H, N, d, seed=11)
    rp, ci, _ = O.mask(q, k, bq, bk, 0.125, 0.3)
    M = _token_mask(rp, ci, B, H, N, bq, bk)
    Os = torch.from_numpy(_full(O.sparse_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq))
    logits = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    lse_all = torch.logsumexp(logits, -1, keepdim=True)
    lse_sel = torch.logsumexp(logits.masked_fill(~M, -math.inf), -1, keepdim=True)
    beta = torch.exp(lse_sel - lse_all)
    rest = _sdpa(q, k, v, ~M)
    dense = _sdpa(q, k, v)
    assert torch.max(torch.abs(beta * Os + (1 - beta) * rest - dense)) < 1e-12


def test_branches_brute_force_token_loops():
    """Pure-Python per-token loops (math.exp, explicit sums) on a tiny case."""
    B, H, N, d, bq, bk = 1, 1, 45, 4, 16, 8
    q, k, v = _qkv(B, H, N, d, seed=5)
    rp, ci, _ = O.mask(q, k, bq, bk, 0.34, 0.5)
    Os = _full(O.sparse_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    Ol = _full(O.linear_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    Q, K, V = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()

    def ph(x):
        return x + 1.0 if x > 0 else math.exp(x)

    for t in range(N):
        i = t // bq
        sel = set(int(j) for j in ci[rp[i]:rp[i + 1]])
        keys_s = [u for u in range(N) if (u // bk) in sel]
        keys_l = [u for u in range(N) if (u // bk) not in sel]
        sc = [sum(Q[t][a] * K[u][a] for a in range(d)) / math.sqrt(d) for u in keys_s]
        mx = max(sc)
        w = [math.exp(s - mx) for s in sc]
        for c in range(d):
            ref = sum(w[n] * V[u][c] for n, u in enumerate(keys_s)) / sum(w)
            assert abs(Os[0, 0, t, c] - ref) < 1e-12
        wl = [sum(ph(Q[t][a]) * ph(K[u][a]) for a in range(d)) for u in keys_l]
        for c in range(d):
            ref = sum(wl[n] * V[u][c] for n, u in enumerate(keys_l)) / sum(wl)
            assert abs(Ol[0, 0, t, c] - ref) < 1e-12


def test_normalisers_brute_force_token_loops():
    """The sparse branch's log-normaliser and the linear branch's
    denominator against pure-Python per-token sums (math.exp, math.log) on a
    tiny case with a ragged last block, an empty row and a full row."""
    B, H, N, d, bq, bk = 1, 1, 45, 4, 16, 8
    q, k, _ = _qkv(B, H, N, d, seed=9)
    Nk = O.n_blocks(N, bk)
    # row 0 lists nothing, row 1 every block, row 2 (ragged) blocks 1, 4, 5
    rp = np.array([0, 0, Nk, Nk + 3])
    ci = np.array(list(range(Nk)) + [1, 4, 5])
    lse = O.sparse_branch_lse(q, k, bq, bk, rp, ci)
    den = O.linear_branch_den(q, k, bq, bk, rp, ci)
    Q, K = q[0, 0].tolist(), k[0, 0].tolist()

    def ph(x):
        return x + 1.0 if x > 0 else math.exp(x)

    for t in range(N):
        i = t // bq
        sel = set(int(j) for j in ci[rp[i]:rp[i + 1]])
        keys_s = [u for u in range(N) if (u // bk) in sel]
        keys_l = [u for u in range(N) if (u // bk) not in sel]
        got_l, got_d = lse[(0, 0, i)][t - i * bq], den[(0, 0, i)][t - i * bq]
        if keys_s:
            ref = math.log(sum(math.exp(sum(Q[t][a] * K[u][a] for a in range(d)) / math.sqrt(d)) for u in keys_s))
            assert abs(got_l - ref) < 1e-12
        else:
            assert got_l == -math.inf
        ref = sum(sum(ph(Q[t][a]) * ph(K[u][a]) for a in range(d)) for u in keys_l)
        assert abs(got_d - ref) <= 1e-12 * max(1.0, ref)


def test_normalisers_recover_the_branches():
    """exp(score - lse) are the sparse branch's weights and phi(q).phi(k) /
    den the linear branch's: both sum to one over their keys and reproduce
    the branch outputs on the 480p workload's first query blocks."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    x = gen.make(wl, heads=1, N=2000)
    rp, ci, _ = O.mask(x.Q, x.K, wl.bq, wl.bk, 0.1, 0.6)
    rows = [(0, 0, 0), (0, 0, 7), (0, 0, O.n_blocks(2000, wl.bq) - 1)]
    lse = O.sparse_branch_lse(x.Q, x.K, wl.bq, wl.bk, rp, ci, rows)
    den = O.linear_branch_den(x.Q, x.K, wl.bq, wl.bk, rp, ci, rows)
    os_ = O.sparse_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, rows)
    ol = O.linear_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp, ci, rows)
    Qd, Kd, Vd = O.as_f64(x.Q)[0, 0], O.as_f64(x.K)[0, 0], O.as_f64(x.V)[0, 0]
    N, d = Qd.shape
    Nk = O.n_blocks(N, wl.bk)
    for (b, h, i) in rows:
        s, e = O.block_range(i, wl.bq, N)
        sel = [int(j) for j in ci[rp[i]:rp[i + 1]]]
        ks = np.concatenate([np.arange(*O.block_range(j, wl.bk, N)) for j in sel])
        kl = np.concatenate([np.arange(*O.block_range(j, wl.bk, N)) for j in range(Nk) if j not in sel])
        P = np.exp(Qd[s:e] @ Kd[ks].T / math.sqrt(d) - lse[(b, h, i)][:, None])
        assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.allclose(P @ Vd[ks], os_[(b, h, i)], rtol=0, atol=1e-12)
        W = O.phi(Qd[s:e]) @ O.phi(Kd[kl]).T / den[(b, h, i)][:, None]
        assert np.allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert np.allclose(W @ Vd[kl], ol[(b, h, i)], rtol=0, atol=1e-12)


def test_combine_endpoints_and_linearity():
    B, H, N, d, bq, bk = 1, 3, 300, 16, 64, 64
    q, k, v = _qkv(B, H, N, d, seed=21)
    rp, ci, _ = O.mask(q, k, bq, bk, 0.2, 0.5)
    a = np.array([0.0, 0.3, 1.0])
    out = _full(O.attn(q, k, v, a, bq, bk, rp, ci), B, H, N, d, bq)
    Os = _full(O.sparse_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    Ol = _full(O.linear_branch(q, k, v, bq, bk, rp, ci), B, H, N, d, bq)
    assert np.array_equal(out[0, 0], Ol[0, 0])
    assert np.array_equal(out[0, 2], Os[0, 2])
    assert np.max(np.abs(out[0, 1] - (0.3 * Os[0, 1] + 0.7 * Ol[0, 1]))) < 1e-14


def test_pool_mean_and_router_linearity():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((1001, 32))
    W = rng.standard_normal((32, 32)) / math.sqrt(32)
    pb = O.pool(X, 64)
    assert pb.shape == (16, 32)
    assert np.max(np.abs(pb[-1] - torch.from_numpy(X[960:]).mean(0).numpy())) < 1e-14
    # pooling then routing == routing every token then pooling
    assert np.max(np.abs(O.route(O.pool(X, 64), W) - O.pool(X @ W, 64))) < 1e-12


def test_mask_invariances():
    """Adding one vector to every pooled key leaves each row's softmax, hence
    the mask, unchanged; permuting whole key blocks permutes the mask."""
    B, H, N, d, bq, bk = 1, 2, 1024, 32, 64, 64
    q, k, v = _qkv(B, H, N, d, seed=8)
    rp, ci, meta = O.mask(q, k, bq, bk, 0.1, 0.6)
    shift = torch.randn(d, dtype=torch.float64, generator=torch.Generator().manual_seed(1))
    rp2, ci2, _ = O.mask(q, k + shift, bq, bk, 0.1, 0.6)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    Nk = meta["Nk"]
    perm = np.random.default_rng(2).permutation(Nk)         # new block b holds old block perm[b]
    kp = k.reshape(B, H, Nk, bk, d)[:, :, perm].reshape(B, H, N, d)
    rp3, ci3, _ = O.mask(q, kp, bq, bk, 0.1, 0.6)
    inv = np.argsort(perm)                                   # old block j is now at inv[j]
    assert np.array_equal(rp, rp3)
    for r in range(len(rp) - 1):
        old = set(ci[rp[r]:rp[r + 1]].tolist())
        new = set(ci3[rp3[r]:rp3[r + 1]].tolist())
        assert new == {int(inv[j]) for j in old}


def test_router_identity_matrices_change_nothing():
    B, H, N, d, bq, bk = 1, 2, 512, 16, 64, 64
    q, k, v = _qkv(B, H, N, d, seed=9)
    I = np.eye(d)
    a = O.mask(q, k, bq, bk, 0.1, 0.6)
    b = O.mask(q, k, bq, bk, 0.1, 0.6, Wq=I, Wk=I)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
