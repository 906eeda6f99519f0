"""Pins of the oracle's single-pass 8-bit sparse branch (SLA2 write-up §三: Q,
K, the attention probabilities and V held in 8 bits, scaled into the 8-bit
range and scaled back; here Q and K as integers, P and V as E4M3
floating-point values of the OCP 8-bit floating-point specification).

Pinned by the format's definition (every bit pattern decoded from sign,
biased exponent and mantissa, checked against hand values; the rounding
function against a brute-force nearest search over that table, ties to the
even mantissa), by the quantisation error bound of a 3-bit mantissa, and by
the bound that ties the single-pass attention to exact float64 softmax
attention on the dequantised inputs: every P code is within 1/16 (relative)
of 256 exp(S - m) or within 2^-10 of it near zero, so each weight moves by at
most that share.  Rows whose running maximum rises several times by large
steps make a missing or wrong rescale fail that bound."""
import math

import numpy as np
import pytest

from oracle import sla_oracle as O


def _table():
    v = O.e4m3_decode(np.arange(256))
    fin = v[np.isfinite(v)]
    return np.unique(fin)  # sorted, +0 and -0 merged


def test_format_hand_values():
    d = O.e4m3_decode
    assert d(0x38) == 1.0             # exponent field 7 = bias: 2^0
    assert d(0x7E) == 448.0           # largest finite: 1.75 * 2^8
    assert d(0x08) == 2.0 ** -6       # smallest normal
    assert d(0x01) == 2.0 ** -9       # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert d(0xB8) == -1.0
    assert d(0x3C) == 1.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    t = _table()
    assert len(t) == 253              # 2 x 126 nonzero finite magnitudes + zero
    assert t.max() == 448.0 and t.min() == -448.0


def test_rounding_matches_brute_force_nearest():
    t = _table()
    pos = t[t >= 0]
    bits = {float(O.e4m3_decode(b)): b for b in range(0x00, 0x7F)}
    # every representable value maps to itself
    assert np.array_equal(O.e4m3(t), t)
    # midpoints go to the neighbour with the even mantissa (lowest bit 0)
    for a, b in zip(pos[:-1], pos[1:]):
        want = a if (bits[float(a)] & 1) == 0 else b
        assert O.e4m3((a + b) / 2) == want, (a, b)
        assert O.e4m3(-(a + b) / 2) == -want
    # random values: the nearest table entry (ties cannot occur here)
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.05, 0.05, 4000),
                        np.exp2(rng.uniform(-12, 8.8, 4000))])
    x = x[np.abs(x) <= 448]
    r = O.e4m3(x)
    dist = np.abs(x[:, None] - t[None, :])
    nearest = t[dist.argmin(axis=1)]
    assert np.array_equal(r, nearest)


def test_channel_quantiser_bound_and_granularity():
    rng = np.random.default_rng(1)
    X = rng.normal(size=(1, 2, 150, 16)).astype(np.float32)
    X[0, 1, :, 3] *= 50.0
    codes, sv = O.quantize_e4m3_channels(X)
    assert sv.shape == (1, 2, 16)
    for h in range(2):
        for c in range(16):
            col = X[0, h, :, c].astype(np.float64)
            assert sv[0, h, c] == np.float32(np.abs(X[0, h, :, c]).max()) / np.float32(448)
            cc = codes[0, h, :, c]
            assert np.abs(cc).max() == 448.0
            assert np.array_equal(O.e4m3(cc), cc)         # every code is an E4M3 value
            # 3 mantissa bits: relative error <= 2^-4 for normals, 2^-10 absolute below
            err = np.abs(cc * float(sv[0, h, c]) - col)
            assert np.all(err <= (2.0 ** -4 * np.abs(col) + 2.0 ** -10 * float(sv[0, h, c])) * (1 + 1e-6))
    zero = np.zeros((1, 1, 64, 8), np.float32)
    z, zs = O.quantize_e4m3_channels(zero)
    assert not z.any() and not zs.any()
    qz = O.quantize_i8f8(X, X, X, 64, 64)
    ref, refs = O.quantize_blocks(X, 64)
    assert np.array_equal(qz["q8"], ref) and np.array_equal(qz["sq"], refs)
    assert np.array_equal(qz["v8"], codes) and np.array_equal(qz["sv"], sv)


def _csr_all(B, H, Nq, Nk, order=None):
    rows = B * H * Nq
    rp = np.arange(rows + 1, dtype=np.int64) * Nk
    ci = np.tile(np.arange(Nk) if order is None else np.asarray(order), rows)
    return rp, ci


def test_equal_scores_give_the_plain_mean():
    # Q = 0: every score is 0, every P code is exactly 256, O = sv * mean(v8)
    rng = np.random.default_rng(2)
    Q = np.zeros((1, 1, 128, 32), np.float32)
    K = rng.normal(size=(1, 1, 256, 32)).astype(np.float32)
    V = rng.normal(size=(1, 1, 256, 32)).astype(np.float32)
    Q2 = np.zeros((1, 1, 256, 32), np.float32)
    Q2[:, :, :128] = Q
    qz = O.quantize_i8f8(Q2, K, V, 128, 64)
    rp, ci = _csr_all(1, 1, 2, 4)
    out, sums = O.sparse_branch_i8f8(qz, 128, 64, rp, ci, with_sums=True)
    want = qz["sv"][0, 0].astype(np.float64) * qz["v8"][0, 0].mean(axis=0)
    np.testing.assert_allclose(out[(0, 0, 0)], np.broadcast_to(want, (128, 32)), rtol=1e-14, atol=0)
    L, m, _ = sums[(0, 0, 0)]
    assert np.all(L == 256.0 * 256) and np.all(m == 0.0)


def _exact_on_dequantised(qz, b, h, i, bq, bk, sel):
    """float64 softmax attention of the dequantised codes over the keys of
    the selected blocks (no 8-bit P)."""
    N, d = qz["q8"].shape[2:]
    s, e = O.block_range(i, bq, N)
    q = qz["q8"][b, h, s:e].astype(np.float64) * float(qz["sq"][b, h, i])
    keys, ks = [], []
    for j in sel:
        a, z = O.block_range(j, bk, N)
        keys.append(np.arange(a, z))
        ks.append(qz["k8"][b, h, a:z].astype(np.float64) * float(qz["sk"][b, h, j]))
    keys = np.concatenate(keys)
    k = np.concatenate(ks)
    v = qz["v8"][b, h, keys] * qz["sv"][b, h].astype(np.float64)[None, :]
    S = q @ k.T / math.sqrt(d)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    return (P / P.sum(axis=1, keepdims=True)) @ v, S


@pytest.mark.parametrize("rising", [False, True])
def test_close_to_exact_attention_with_a_rising_maximum(rising):
    """The result is a weighted mean of the values whose weights differ from
    softmax(S) only by the P rounding: each code is within 2^-4 (relative) or
    2^-10 (absolute, near 0) of 256 exp(S - m), so the output moves by at most
    max|v| * 2 * (2^-4 + 2^-10 * n / L) per element.  With `rising`, the
    blocks come in increasing order of their score level (the running maximum
    rises at every unit by several units of S), which a missing or wrong
    rescale of the earlier units would turn into errors far above the bound."""
    rng = np.random.default_rng(3)
    B, H, N, d, bq, bk = 1, 2, 640, 64, 64, 64
    Q = rng.normal(size=(B, H, N, d)).astype(np.float32)
    K = rng.normal(size=(B, H, N, d)).astype(np.float32)
    V = rng.normal(size=(B, H, N, d)).astype(np.float32)
    if rising:
        # key block j leans toward the queries with a weight growing in j
        qdir = Q.mean(axis=2, keepdims=True)
        for j in range(N // bk):
            K[:, :, j * bk:(j + 1) * bk] += (0.6 * j) * qdir / np.linalg.norm(qdir) * math.sqrt(d)
    qz = O.quantize_i8f8(Q, K, V, bq, bk)
    Nq, Nk = N // bq, N // bk
    rp, ci = _csr_all(B, H, Nq, Nk)
    rows = [(0, h, i) for h in range(H) for i in range(Nq)]
    out, sums = O.sparse_branch_i8f8(qz, bq, bk, rp, ci, rows=rows, with_sums=True)
    worst = 0.0
    rises = 0
    for (b, h, i) in rows:
        exact, Sx = _exact_on_dequantised(qz, b, h, i, bq, bk, range(Nk))
        L, m, _ = sums[(b, h, i)]
        vmax = np.abs(qz["v8"][b, h] * qz["sv"][b, h].astype(np.float64)[None, :]).max(axis=0)
        n = Sx.shape[1]
        bound = vmax[None, :] * 2 * (2.0 ** -4 + 2.0 ** -10 * n / L[:, None]) * (1 + 1e-9)
        err = np.abs(out[(b, h, i)] - exact)
        assert np.all(err <= bound), (h, i, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
        assert np.all(np.isfinite(m)) and np.allclose(m, Sx.max(axis=1), rtol=1e-5, atol=1e-6)
        unit_max = Sx.reshape(Sx.shape[0], Nk, bk).max(axis=2)
        rises += int((np.diff(np.maximum.accumulate(unit_max, axis=1), axis=1) > 1.0).sum())
    if rising:
        assert rises > 500  # the running maximum really moves, by more than 1 in S
    assert worst < 0.5


def test_first_unit_holding_the_maximum_needs_no_rescale():
    """When the first unit of every row already holds the row maximum, no
    rescale happens and the result is the sum over all keys of the codes
    taken against that maximum (f8_p_codes over the whole row in one
    product), exactly."""
    rng = np.random.default_rng(4)
    B, H, N, d, bq, bk = 1, 1, 256, 32, 64, 64
    u = np.full(d, 3.0 / math.sqrt(d))                   # every query leans along u
    Q = (u + 0.3 * rng.normal(size=(B, H, N, d))).astype(np.float32)
    K = (0.3 * rng.normal(size=(B, H, N, d))).astype(np.float32)
    K[:, :, :bk] += (2.0 * u).astype(np.float32)          # so block 0 scores highest for every query
    V = rng.normal(size=(B, H, N, d)).astype(np.float32)
    qz = O.quantize_i8f8(Q, K, V, bq, bk)
    rp, ci = _csr_all(B, H, N // bq, N // bk)
    out, sums = O.sparse_branch_i8f8(qz, bq, bk, rp, ci, with_sums=True)
    lam = np.float32(1.0 / math.sqrt(d))
    l2e = np.float32(math.log2(math.e))
    for i in range(N // bq):
        s, e = O.block_range(i, bq, N)
        c = [np.float32(np.float32(qz["sq"][0, 0, i] * qz["sk"][0, 0, j]) * lam) for j in range(N // bk)]
        I = qz["q8"][0, 0, s:e].astype(np.int64) @ qz["k8"][0, 0].astype(np.int64).T
        R = I.astype(np.float32)
        Sb = [(R[:, j * bk:(j + 1) * bk] * c[j]).astype(np.float32).max(axis=1) for j in range(N // bk)]
        assert np.all(Sb[0] >= np.max(Sb, axis=0))
        m = Sb[0]
        b = ((m * l2e).astype(np.float32) - np.float32(8)).astype(np.float32)
        a = np.concatenate([np.full(bk, np.float32(cj * l2e), np.float32) for cj in c])
        p8 = O.f8_p_codes(R, a[None, :], b[:, None])
        want = qz["sv"][0, 0].astype(np.float64)[None, :] * (p8 @ qz["v8"][0, 0]) / p8.sum(axis=1)[:, None]
        np.testing.assert_allclose(out[(0, 0, i)], want, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(sums[(0, 0, i)][0], p8.sum(axis=1), rtol=1e-13)


_U = 2.0 ** -24  # float32 unit roundoff


def _midpoint_distance(x):
    """Distance of x >= 0 to the nearest midpoint between E4M3 neighbours."""
    _, e = np.frexp(x)
    step = np.ldexp(1.0, (np.maximum(e - 1, -6) - 3).astype(np.int64))
    return np.abs(x - (np.floor(x / step) + 0.5) * step), step


def test_float32_codes_match_the_definition_on_the_480p_sample():
    """On the 480p SLA2 workload (two heads, the oracle's own mask), every P
    code f8_p_codes forms for 16 sampled row blocks equals E4M3(256 exp(S -
    m)) evaluated in float64 (S = fl32(I c), m the same running maximum),
    except where that value lies within the float32 error bound of an E4M3
    midpoint; those few differ by one E4M3 step.  Bound on the relative error
    of the float32 value: each rounding adds at most u |value| (u = 2^-24) to
    t in log2 units: a and fl32(log2 e) (2 u log2(e) |I c|), fl32(m log2 e)
    (2 u log2(e) |m|), b (u |b|), t (u |t|); then 2^E - 1 <= E ln 2 (1 + E),
    plus u for rounding 2^t; doubled for slack."""
    import gen
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    x = gen.make(wl, heads=2)
    rp, ci, _ = O.mask(x.Q, x.K, wl.bq, wl.bk, wl.k_frac, wl.p, keep_info=False)
    qz = O.quantize_i8f8(x.Q, x.K, x.V, wl.bq, wl.bk)
    q8, k8 = qz["q8"].astype(np.int64), qz["k8"].astype(np.int64)
    lam = np.float32(1.0 / math.sqrt(wl.d))
    l2e = np.float32(math.log2(math.e))
    L2 = math.log2(math.e)
    rng = np.random.default_rng(0)
    rows = [(h, int(i)) for h in range(2) for i in rng.choice(wl.Nq, 8, replace=False)]
    rows[-1] = (1, wl.Nq - 1)
    total = excused = 0
    for h, i in rows:
        r = h * wl.Nq + i
        s, e = O.block_range(i, wl.bq, wl.N)
        m = np.full(e - s, -np.inf, dtype=np.float32)
        for j in ci[rp[r]:rp[r + 1]]:
            ks, ke = O.block_range(int(j), wl.bk, wl.N)   # bk = 64: one unit per block
            c = np.float32(np.float32(qz["sq"][0, h, i] * qz["sk"][0, h, j]) * lam)
            I = q8[0, h, s:e] @ k8[0, h, ks:ke].T
            S = (I.astype(np.float32) * c).astype(np.float32)
            m = np.maximum(m, S.max(axis=1))
            b = ((m * l2e).astype(np.float32) - np.float32(8)).astype(np.float32)
            got = O.f8_p_codes(I.astype(np.float32), np.float32(c * l2e), b[:, None])
            xv = 256.0 * np.exp(S.astype(np.float64) - m.astype(np.float64)[:, None])
            want = O.e4m3(xv)
            t = np.log2(np.maximum(xv, 1e-300))
            Ic = np.abs(I * np.float64(c))
            E = _U * (2 * L2 * Ic + L2 * np.abs(S.astype(np.float64))
                      + 2 * L2 * np.abs(m.astype(np.float64))[:, None]
                      + np.abs(b.astype(np.float64))[:, None] + np.abs(t))
            bound = 2.0 * xv * (E * math.log(2.0) * (1 + E) + _U)
            dist, step = _midpoint_distance(xv)
            diff = got != want
            assert np.all(dist[diff] <= bound[diff]), (h, i)
            assert np.all(np.abs(got - want) <= step * (1 + 1e-12) + 1e-300)
            total += got.size
            excused += int(diff.sum())
    assert total > 100000
    print(f"codes {total}, differing from the float64 value {excused}")
    assert excused <= 1e-3 * total, (excused, total)


def test_empty_row_and_partial_units():
    rng = np.random.default_rng(5)
    B, H, N, d, bq, bk = 1, 1, 200, 32, 64, 128   # bk = 128: two units per block; last block 72 keys
    Q, K, V = (rng.normal(size=(B, H, N, d)).astype(np.float32) for _ in range(3))
    qz = O.quantize_i8f8(Q, K, V, bq, bk)
    Nq = O.n_blocks(N, bq)
    rp = np.array([0, 0, 1, 3, 4], np.int64)          # row 0 empty
    ci = np.array([1, 0, 1, 0], np.int64)
    out = O.sparse_branch_i8f8(qz, bq, bk, rp, ci)
    assert not out[(0, 0, 0)].any()
    for i, sel in ((1, [1]), (2, [0, 1]), (3, [0])):
        exact, Sx = _exact_on_dequantised(qz, 0, 0, i, bq, bk, sel)
        vmax = np.abs(qz["v8"][0, 0] * qz["sv"][0, 0].astype(np.float64)[None, :]).max(axis=0)
        assert np.all(np.abs(out[(0, 0, i)] - exact) <= vmax * 2 * (2.0 ** -4 + 2.0 ** -10 * Sx.shape[1]))
    assert out[(0, 0, 3)].shape == (200 - 192, d)
