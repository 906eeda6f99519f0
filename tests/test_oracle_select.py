"""Pins of the oracle's selection rules against brute-force enumeration and
hand-worked examples (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import sla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "selection_examples.json")


def _lexkey(P, subset):
    """Sort key of a subset under the shared order (P desc, index asc)."""
    return sorted(((-P[j], j) for j in subset))


def brute_topk(P, k):
    """The k-subset with the largest total mass; among equal totals the one
    whose ordered members come first (ties to the lower index)."""
    best = None
    for sub in itertools.combinations(range(len(P)), k):
        tot = sum(P[j] for j in sub)
        key = (-tot, _lexkey(P, sub))
        if best is None or key < best[0]:
            best = (key, sub)
    return sorted(best[1])


def brute_topp(P, p):
    """The feasible set (total >= p) of fewest members; among those the one of
    largest mass, then the one whose ordered members come first."""
    if p <= 0:
        return []
    Nk = len(P)
    for n in range(1, Nk + 1):
        cands = []
        for sub in itertools.combinations(range(Nk), n):
            tot = sum(P[j] for j in sub)  # exact: dyadic weights
            if tot >= p:
                cands.append(((-tot, _lexkey(P, sub)), sub))
        if cands:
            return sorted(min(cands)[1])
    return list(range(Nk))


def _dyadic_probs(rng, Nk, denom=1024, ties=False):
    if ties:
        w = rng.integers(1, 4, size=Nk)
    else:
        w = rng.permutation(np.arange(1, 4 * Nk + 1))[:Nk]
    # normalise to integer weights summing to denom (exact dyadic probabilities)
    w = np.floor(w / w.sum() * denom).astype(np.int64)
    w[0] += denom - w.sum()
    w = np.maximum(w, 0)
    return w / float(denom)


@pytest.mark.parametrize("Nk", [1, 2, 5, 8, 11])
@pytest.mark.parametrize("ties", [False, True])
def test_union_matches_brute_force(Nk, ties):
    rng = np.random.default_rng(100 + Nk + 7 * ties)
    for trial in range(12):
        P = _dyadic_probs(rng, Nk, ties=ties)
        assert abs(P.sum() - 1.0) == 0.0
        k = int(rng.integers(0, Nk + 1))
        p = float(rng.integers(0, 1025)) / 1024.0  # exactly representable in fp32
        sel, info = O.select_row(P, k, p)
        tk = brute_topk(P, k)
        tp = brute_topp(P, p)
        assert sorted(info["order"][:info["k"]]) == tk
        assert sorted(info["order"][:info["kp"]]) == tp
        assert list(sel) == sorted(set(tk) | set(tp))


def test_golden_examples_from_the_pages():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        P = np.array(c["weights"], dtype=np.float64) / c["denom"]
        sel, info = O.select_row(P, c["k"], c["p"])
        assert sorted(info["order"][:info["k"]].tolist()) == c["topk"], c["name"]
        assert sorted(info["order"][:info["kp"]].tolist()) == c["topp"], c["name"]
        assert sel.tolist() == c["union"], c["name"]


@pytest.mark.parametrize("k_frac,Nk,expect", [
    (0.03, 512, 16), (0.05, 512, 26), (0.1, 16, 2), (0.04, 1182, 48), (0.03, 100, 3),
    (0.5, 2, 1), (0.0, 512, 0), (1.0, 512, 512), (0.25, 4, 1), (1e-6, 7, 1)])
def test_k_from_frac(k_frac, Nk, expect):
    assert O.k_from_frac(k_frac, Nk) == expect


def test_uniform_topp_keeps_ceil_p_n():
    """Uniform P over Nk=16 (dyadic): Top-p keeps ceil(p*Nk) blocks, the
    lowest indices first."""
    P = np.full(16, 1.0 / 16)
    for p in (0.0625, 0.25, 0.3, 0.5, 0.75, 0.99, 1.0):
        _, info = O.select_row(P, 0, p)
        p32 = float(np.float32(p))
        assert info["kp"] == int(np.ceil(p32 * 16 - 1e-12)) if p32 * 16 <= 16 else 16
        assert list(info["order"][:4]) == [0, 1, 2, 3]


def test_sparsity_of_the_stated_workloads():
    """The 480p workloads state about 90% block sparsity for k_frac=0.05, p=0.9
    and about 97% for k_frac=0.03, p=0.5.  Under the oracle's readings (1/sqrt(d)
    scale, ceil k, inclusive Top-p) two heads of each reproduce that."""
    import gen
    for name, lo, hi in (("video480p-sparse-N32760", 0.85, 0.96),
                         ("video480p-sla2-N32760", 0.95, 0.985)):
        wl = gen.WORKLOADS[name]
        x = gen.make(wl, heads=2)
        rp, ci, meta = O.mask(x.Q, x.K, wl.bq, wl.bk, wl.k_frac, wl.p, keep_info=False)
        sparsity = 1.0 - len(ci) / float(2 * wl.Nq * wl.Nk)
        assert lo <= sparsity <= hi, (name, sparsity)
