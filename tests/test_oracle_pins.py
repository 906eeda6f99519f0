"""Pins of two oracle choices that no worked example on the pages fixes
(CPU only).

1. The 1/sqrt(d) scale of the pooled block logits.  The pages print only the
   textbook attention formula softmax(Q K^T / sqrt(d)) V (the explainer page
   "清华SpargeAttention2技术解析：如何让AI视频生成提速16倍", section 3 on the
   implementation principle); the pooled logits take the same scale.  What decides
   between "scaled" and "unscaled" is the stated behaviour of the 480p
   sparse-only workload: k_frac = 0.05 and p = 0.9 are said to give about 90%
   block sparsity.  Top-k alone keeps ceil(0.05 * 512) = 26 of 512 blocks
   (94.9% sparsity), so "about 90%" needs Top-p to add blocks on a large
   share of rows - the hybrid rule of the SpargeAttention2 write-up §一 doing
   its job.  With the scale it does (93% sparsity, Top-p deciding most rows);
   without it the pooled maps are so peaked that Top-p never adds a block and
   the sparsity is Top-k's 94.9%.  The test below asserts the scaled
   behaviour, and a second test plants the unscaled logits in the oracle and
   requires the same check to fail.

2. The 8-bit branch's P codes (SLA2 write-up §三).  Their definition is
   code = round-half-even(127 exp(S - m)) of the float32 scores S; the oracle
   takes that integer decision in float32 (as exp2 of one fused
   multiply-add), the precision the kernel decides it in.  The test compares
   those codes with the definition evaluated in float64 and allows a
   difference only where 127 exp(S - m) lies within the float32 evaluation's
   own error bound of a half-integer, where float32 cannot decide the
   rounding.
"""
import math

import numpy as np

import gen
from oracle import sla_oracle as O

C2 = "video480p-sparse-N32760"


def _c2_selection_stats(oracle_mod, heads=2):
    """Sparsity and the share of rows whose count Top-p decides (kp > k) on
    the first heads of the 480p sparse-only workload."""
    wl = gen.WORKLOADS[C2]
    x = gen.make(wl, heads=heads)
    rp, ci, meta = oracle_mod.mask(x.Q, x.K, wl.bq, wl.bk, wl.k_frac, wl.p)
    rows = meta["rows"]
    topp_rows = sum(1 for r in rows if r["kp"] > r["k"]) / len(rows)
    sparsity = 1.0 - len(ci) / float(heads * wl.Nq * wl.Nk)
    return sparsity, topp_rows, meta["k"]


def _stated_behaviour(sparsity, topp_rows, k, Nk=512):
    """"About 90%" block sparsity with k = 26 of 512: strictly below the
    94.9% Top-k alone gives (Top-p adds blocks), on at least 40% of rows."""
    topk_only = 1.0 - k / float(Nk)
    return 0.88 <= sparsity <= 0.945 and sparsity < topk_only - 0.005 and topp_rows >= 0.4


def test_topp_adds_blocks_at_the_stated_90_percent_workload():
    sparsity, topp_rows, k = _c2_selection_stats(O)
    assert k == 26
    assert _stated_behaviour(sparsity, topp_rows, k), (sparsity, topp_rows)


def test_unscaled_pooled_logits_fail_the_same_check(monkeypatch):
    """Plant the unscaled reading in the oracle: the check above must fail."""
    def unscaled(qhat, khat):
        return qhat @ khat.T

    monkeypatch.setattr(O, "block_scores", unscaled)
    sparsity, topp_rows, k = _c2_selection_stats(O)
    assert topp_rows < 0.05, topp_rows          # Top-p never adds a block
    assert not _stated_behaviour(sparsity, topp_rows, k), (sparsity, topp_rows)


# ----------------------------------------------------------- 8-bit P codes
_U = 2.0 ** -24  # float32 unit roundoff


def _definition_codes(S: np.ndarray, m: np.float32):
    """round-half-even(127 exp(S - m)) in float64, and 127 exp(S - m)."""
    x = 127.0 * np.exp(S.astype(np.float64) - float(m))
    return np.rint(x), x


def _float32_error_bound(I, c, S, m, x):
    """Bound on |p - x| for the oracle's float32 evaluation p of x = 127
    exp(S - m): p = fl32(2^t), t = fl32(I a - b), a = fl32(c fl32(log2 e)),
    b = fl32(fl32(m fl32(log2 e)) - fl32(log2 127)).  Each float32 rounding
    contributes at most u |value| (u = 2^-24) to t in log2 units:
      a and fl32(log2 e):   2 u log2(e) |I c|,  S = fl32(I c):  u log2(e) |S|
      fl32(m log2 e), b:    2 u log2(e) |m| + u |b|,  fl32(log2 127):  u log2 127
      t itself:             u |t|
    and the float64 steps add < 2^-50 (|I a| + |b|).  Then x's relative error
    is 2^E - 1 <= E ln 2 (1 + E), plus u for rounding 2^t to float32.  The
    bound is doubled for slack."""
    L = math.log2(math.e)
    t = np.log2(np.maximum(x, 1e-300))
    Ic = np.abs(I.astype(np.float64) * c.astype(np.float64))
    b = abs(float(m)) * L - math.log2(127.0)
    E = _U * (2 * L * Ic + L * np.abs(S.astype(np.float64)) + 2 * L * abs(float(m)) + abs(b)
              + math.log2(127.0) + np.abs(t)) + 2.0 ** -50 * (Ic * L + abs(b))
    rel = E * math.log(2.0) * (1 + E) + _U
    return 2.0 * x * rel


def test_p_codes_match_the_definition_on_the_480p_sample():
    """On the 480p SLA2 workload (two heads), every P code the oracle forms
    for 16 sampled row blocks equals round-half-even(127 exp(S - m)) except
    where that value lies within the float32 error bound of a half-integer;
    those few differ by exactly one."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    x = gen.make(wl, heads=2)
    rp, ci, _ = O.mask(x.Q, x.K, wl.bq, wl.bk, wl.k_frac, wl.p, keep_info=False)
    qz = O.quantize_i8(x.Q, x.K, x.V, wl.bq, wl.bk)
    q8, k8 = qz["q8"].astype(np.int64), qz["k8"].astype(np.int64)
    lam = np.float32(1.0 / math.sqrt(wl.d))
    rng = np.random.default_rng(0)
    rows = [(h, int(i)) for h in range(2) for i in rng.choice(wl.Nq, 8, replace=False)]
    rows[-1] = (1, wl.Nq - 1)  # the partial last query block
    total = excused = 0
    for h, i in rows:
        r = h * wl.Nq + i
        sel = ci[rp[r]:rp[r + 1]]
        keys = np.concatenate([np.arange(*O.block_range(int(j), wl.bk, wl.N)) for j in sel])
        c = np.concatenate([np.full(O.block_range(int(j), wl.bk, wl.N)[1] - O.block_range(int(j), wl.bk, wl.N)[0],
                                    np.float32(np.float32(qz["sq"][0, h, i] * qz["sk"][0, h, j]) * lam),
                                    dtype=np.float32) for j in sel])
        s, e = O.block_range(i, wl.bq, wl.N)
        I = q8[0, h, s:e] @ k8[0, h, keys].T
        S = (I.astype(np.float32) * c[None, :]).astype(np.float32)
        for t in range(e - s):
            m = S[t].max()
            got = O.p_codes(I[t], c, m)
            want, xv = _definition_codes(S[t], m)
            bound = _float32_error_bound(I[t], c, S[t], m, xv)
            diff = got != want
            near_half = np.abs(xv - (np.floor(xv) + 0.5)) <= bound
            assert np.all(near_half[diff]), (h, i, t, xv[diff & ~near_half][:4])
            assert np.all(np.abs(got - want) <= 1)
            total += len(got)
            excused += int(diff.sum())
    assert total > 100000
    # the float32 decision differs from the float64 one only rarely
    assert excused <= 1e-4 * total, (excused, total)
