"""sla_mask_noalloc (the mask with the library's static device scratch, for
callers that cannot allocate) against sla_mask with a caller workspace:
identical CSR, entry for entry, on two calls in a row - the second with a
smaller problem, so it runs on what the first left in the shared scratch -
and the size limit is refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from tests import _util as U

pytestmark = pytest.mark.gpu


def _inputs(wl):
    x = gen.make(wl)
    return x, U.dev(x.Q, x.K), U.dev(x.Wq, x.Wk)


def _same(x, qk, wqk, k_frac, p):
    (q, k), (wq, wk) = qk, wqk
    wl = x.wl
    rp0, ci0 = S.sla_mask(q, k, wl.bq, wl.bk, k_frac, p, wq, wk)
    rp1 = torch.full_like(rp0, -7)
    ci1 = torch.full_like(ci0, -7)
    S.sla_mask_noalloc(q, k, wl.bq, wl.bk, k_frac, p, wq, wk, row_ptr=rp1, col_idx=ci1)
    torch.cuda.synchronize()
    n = int(rp0[-1])
    assert torch.equal(rp0, rp1), "row_ptr differs"
    assert torch.equal(ci0[:n], ci1[:n]), "col_idx differs"
    assert bool((ci1[n:] == -7).all()), "entries past nnz written"
    return n


def test_noalloc_matches_sla_mask_twice_then_smaller():
    big = gen.WORKLOADS["video480p-sla2-N32760"]
    small = gen.Workload("adhoc", B=2, H=3, grid=(1, 1, 5001), d=64, bq=64, bk=128, k_frac=0.1, p=0.7,
                         dtype="bf16", router=True, seed=23)
    print("[noalloc] 480p SLA2 workload, twice", flush=True)
    xb = _inputs(big)
    prob = S.problem(xb[1][0], big.bq, big.bk)
    need = S.sla_mask_noalloc_bytes(prob, S.select(big.k_frac, big.p))
    assert 0 < need <= S.NOALLOC_SCRATCH_BYTES
    n1 = _same(xb[0], xb[1], xb[2], big.k_frac, big.p)
    n2 = _same(xb[0], xb[1], xb[2], big.k_frac, big.p)
    assert n1 == n2 > 0
    print(f"[noalloc] smaller routed problem (scratch {need} bytes before)", flush=True)
    xs = _inputs(small)
    _same(xs[0], xs[1], xs[2], small.k_frac, small.p)
    print("[noalloc] fp32 tiny workload", flush=True)
    xt = _inputs(gen.WORKLOADS["tiny-fp32-N1024"])
    _same(xt[0], xt[1], xt[2], 0.1, 0.6)


def test_noalloc_refuses_problems_beyond_its_scratch():
    """The 720p workload's mask scratch (its pooled logits alone are 224 MB)
    exceeds the static array: refused on the host before any launch."""
    L = S.lib()
    wl = gen.WORKLOADS["video720p-sla2-N75600"]
    p = S.Problem(wl.B, wl.H, wl.N, wl.d, wl.bq, wl.bk, S.SLA_BF16)
    sel = S.Select(wl.k_frac, wl.p, None, None)
    assert L.sla_mask_noalloc_bytes(ctypes.byref(p), ctypes.byref(sel)) > S.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    cap = L.sla_mask_capacity(ctypes.byref(p))
    assert L.sla_mask_noalloc(ctypes.byref(p), ctypes.byref(sel), fake, fake, fake, fake, cap, None) == -6
