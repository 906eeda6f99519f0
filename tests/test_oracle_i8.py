"""Pins of the oracle's 8-bit sparse branch (SLA2 write-up §三: Q, K, the
attention probabilities and V held as 8-bit integers, scaled into the 8-bit
range and scaled back).

Pinned by hand-computed examples (quantiser ties, scores with a known
exponential, per-block scale indexing), by the quantisation error bound
|x - s code| <= s / 2, and by the bound that ties the integer attention to
the exact float64 sparse branch on the dequantised inputs: every P code is
within 1/2 of 127 exp(S - m), so the weights move by at most n / sum(code)
in L1 and each output by at most max|v| times that."""
import math

import numpy as np
import pytest

from oracle import sla_oracle as O


def test_quantiser_hand_example():
    # amax 1: reciprocal 127 exactly; 0.5 * 127 = 63.5 is a tie (-> 64, even),
    # 0.25 * 127 = 31.75 -> 32
    x = np.array([[0.5, -1.0], [0.25, 0.0]], dtype=np.float32)
    codes, s = O.quant_codes(x, np.abs(x).max())
    assert codes.tolist() == [[64, -127], [32, 0]]
    assert s == np.float32(1.0) / np.float32(127.0)


def test_quantiser_zero_block_and_bound():
    codes, s = O.quant_codes(np.zeros((3, 4), np.float32), 0.0)
    assert s == 0 and not codes.any()
    rng = np.random.default_rng(0)
    x = (rng.normal(size=(64, 128)) * 3).astype(np.float32)
    codes, s = O.quant_codes(x, np.abs(x).max())
    err = np.abs(x.astype(np.float64) - float(s) * codes)
    assert err.max() <= float(s) * 0.5 * (1 + 1e-5)
    assert np.abs(codes).max() == 127
    assert codes.flat[np.abs(x).argmax()] == 127 * np.sign(x.flat[np.abs(x).argmax()])


def test_block_and_channel_granularity():
    rng = np.random.default_rng(1)
    X = rng.normal(size=(1, 2, 70, 8)).astype(np.float32)
    X[0, 1, 64:] *= 100.0                  # second block of head 1 much larger
    codes, sc = O.quantize_blocks(X, 64)
    assert sc.shape == (1, 2, 2)
    assert sc[0, 1, 1] == np.float32(np.abs(X[0, 1, 64:]).max()) / np.float32(127)
    assert sc[0, 1, 0] == np.float32(np.abs(X[0, 1, :64]).max()) / np.float32(127)
    vc, vs = O.quantize_channels(X)
    assert vs.shape == (1, 2, 8)
    for c in range(8):
        assert vs[0, 1, c] == np.float32(np.abs(X[0, 1, :, c]).max()) / np.float32(127)


def _hand_qz(sk1=1.0, k2=(2, 2, 0, 0)):
    return {
        "q8": np.ones((1, 1, 3, 4), np.int8), "sq": np.ones((1, 1, 1), np.float32),
        "k8": np.array([[1, 1, 1, 1], [1, 1, 0, 0], list(k2)], np.int8)[None, None],
        "sk": np.array([1.0, sk1], np.float32)[None, None],
        "v8": np.array([[10, 0, 0, 0], [0, 127, 0, 0], [-10, 0, 5, 0]], np.int8)[None, None],
        "sv": np.array([0.125, 0.0078125, 1.0, 0.0], np.float32)[None, None],
    }


@pytest.mark.parametrize("sk1,k2", [(1.0, (2, 2, 0, 0)), (0.5, (4, 4, 0, 0))])
def test_integer_attention_hand_example(sk1, k2):
    # d = 4: 1/sqrt(d) = 0.5 exactly.  Scores: key 0 I = 4 -> S = 2, key 1
    # I = 2 -> S = 1, key 2 (second key block, scale sk1) S = 2 either way.
    # m = 2, codes 127, round(127/e) = round(46.72) = 47, 127; sum 301.
    qz = _hand_qz(sk1, k2)
    out = O.sparse_branch_i8(qz, 4, 2, np.array([0, 2]), np.array([0, 1]))[(0, 0, 0)]
    want = np.array([0.125 * (127 * 10 - 127 * 10), 0.0078125 * 47 * 127, 127 * 5, 0.0]) / 301
    np.testing.assert_allclose(out, np.tile(want, (3, 1)), rtol=0, atol=1e-15)


def test_integer_attention_selects_blocks():
    # only key block 1 (key 2) selected: a single key, weight 1
    qz = _hand_qz()
    out = O.sparse_branch_i8(qz, 4, 2, np.array([0, 1]), np.array([1]))[(0, 0, 0)]
    np.testing.assert_allclose(out[0], [0.125 * -10, 0.0, 5.0, 0.0], atol=1e-15)
    empty = O.sparse_branch_i8(qz, 4, 2, np.array([0, 0]), np.array([], dtype=np.int64))[(0, 0, 0)]
    assert not empty.any()


def test_p_codes_range_and_max():
    rng = np.random.default_rng(2)
    I = rng.integers(-20000, 20000, size=500)
    c = np.full(500, np.float32(3e-4), np.float32)
    S = (I.astype(np.float32) * c).astype(np.float32)
    codes = O.p_codes(I, c, S.max())
    assert codes[np.argmax(I)] == 127
    exact = 127 * np.exp(S.astype(np.float64) - float(S.max()))
    assert np.abs(codes - exact).max() <= 0.5 + 1e-4


def _case(seed, N, d, bq, bk, density):
    rng = np.random.default_rng(seed)
    Q = rng.normal(size=(1, 2, N, d)).astype(np.float32) * 2
    K = rng.normal(size=(1, 2, N, d)).astype(np.float32)
    V = rng.normal(size=(1, 2, N, d)).astype(np.float32)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    rp, ci = [0], []
    for r in range(2 * Nq):
        sel = np.flatnonzero(rng.random(Nk) < density)
        ci.extend(sel.tolist())
        rp.append(len(ci))
    return Q, K, V, np.array(rp), np.array(ci, dtype=np.int64)


@pytest.mark.parametrize("seed,N,d,bq,bk,density", [(3, 200, 16, 32, 16, 0.5), (4, 130, 32, 64, 32, 0.3)])
def test_close_to_exact_branch_on_dequantised_inputs(seed, N, d, bq, bk, density):
    """Against the float64 sparse branch on sq q8, sk k8, sv v8: the only
    difference left is the P rounding, bounded per output by
    max|v| * n / (sum_j 127 P_j - n / 2)."""
    Q, K, V, rp, ci = _case(seed, N, d, bq, bk, density)
    qz = O.quantize_i8(Q, K, V, bq, bk)
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    Qd = qz["q8"] * np.repeat(qz["sq"], bq, axis=2)[:, :, :N, None].astype(np.float64)
    Kd = qz["k8"] * np.repeat(qz["sk"], bk, axis=2)[:, :, :N, None].astype(np.float64)
    Vd = qz["v8"] * qz["sv"][:, :, None, :].astype(np.float64)
    got = O.sparse_branch_i8(qz, bq, bk, rp, ci)
    ref = O.sparse_branch(Qd, Kd, Vd, bq, bk, rp, ci)
    checked = 0
    for key, o in got.items():
        b, h, i = key
        r = (b * 2 + h) * Nq + i
        sel = ci[rp[r]:rp[r + 1]]
        if len(sel) == 0:
            assert not o.any()
            continue
        keys = np.concatenate([np.arange(*O.block_range(int(j), bk, N)) for j in sel])
        s, e = O.block_range(i, bq, N)
        Sx = Qd[b, h, s:e] @ Kd[b, h, keys].T / math.sqrt(d)
        P = np.exp(Sx - Sx.max(axis=1, keepdims=True))
        n = len(keys)
        bound = np.abs(Vd[b, h, keys]).max() * n / (127 * P.sum(axis=1) - n / 2)
        assert np.all(np.abs(o - ref[key]) <= bound[:, None] + 1e-12)
        checked += 1
    assert checked > 0


def test_block_order_and_power_of_two_scaling():
    Q, K, V, rp, ci = _case(5, 150, 16, 32, 16, 0.4)
    qz = O.quantize_i8(Q, K, V, 32, 16)
    base = O.sparse_branch_i8(qz, 32, 16, rp, ci)
    # the definition does not depend on the order of a row's blocks
    ci_rev = ci.copy()
    for r in range(len(rp) - 1):
        ci_rev[rp[r]:rp[r + 1]] = ci[rp[r]:rp[r + 1]][::-1]
    rev = O.sparse_branch_i8(qz, 32, 16, rp, ci_rev)
    for k in base:
        np.testing.assert_array_equal(base[k], rev[k])
    # V scaled by 4: identical codes, scales x4, outputs x4 exactly
    qz4 = O.quantize_i8(Q, K, V * 4, 32, 16)
    np.testing.assert_array_equal(qz4["v8"], qz["v8"])
    np.testing.assert_array_equal(qz4["sv"], qz["sv"] * 4)
    four = O.sparse_branch_i8(qz4, 32, 16, rp, ci)
    for k in base:
        np.testing.assert_array_equal(four[k], base[k] * 4)
