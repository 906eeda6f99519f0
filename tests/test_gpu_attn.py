"""GPU parity of the attention entry points against the oracle, with the GPU's
own mask fed to the oracle.  Bars: fp32 max-abs <= 1e-5; bf16 max-abs <= 2e-2
and relative L1 (sum |O - O_ref| / sum |O_ref|) <= 5e-3."""
import dataclasses

import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

F32_MAXABS = 1e-5
BF16_MAXABS, BF16_REL = 2e-2, 5e-3


def _bar(dtype, maxabs, rel, what):
    if dtype == "fp32":
        assert maxabs <= F32_MAXABS, f"{what}: max-abs {maxabs:.3g}"
    else:
        assert maxabs <= BF16_MAXABS and rel <= BF16_REL, f"{what}: max-abs {maxabs:.3g} rel {rel:.3g}"


def _adhoc(dtype, N, d, bq, bk, k_frac, p, seed=11, B=2, H=3, alpha=None):
    wl = gen.Workload("adhoc", B=B, H=H, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=k_frac, p=p,
                      dtype=dtype, alpha=alpha or (), alpha_range=(0.3, 0.9), seed=seed)
    return gen.make(wl)


def _run_all(x, rows=None):
    """Mask + every entry point; returns GPU outputs and the oracle's on
    `rows` (a list of (b, h, i), a function of the GPU's row_ptr returning
    one, or None for every row)."""
    wl = x.wl
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    wq, wk = U.dev(x.Wq, x.Wk)
    o, rp, ci = S.sla_attn_fwd(q, k, v, a, wl.bq, wl.bk, wl.k_frac, wl.p, wq, wk)
    os_ = S.sla_sparse_fwd(q, k, v, wl.bq, wl.bk, rp, ci)
    ol = S.sla_linear_fwd(q, k, v, wl.bq, wl.bk, rp, ci)
    torch.cuda.synchronize()
    rp_g, ci_g = U.csr(rp, ci)
    B, H, N, d = x.Q.shape
    Nq = O.n_blocks(N, wl.bq)
    if callable(rows):
        rows = rows(rp_g)
    rows = rows or [(b, h, i) for b in range(B) for h in range(H) for i in range(Nq)]
    ref_s = O.sparse_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp_g, ci_g, rows)
    ref_l = O.linear_branch(x.Q, x.K, x.V, wl.bq, wl.bk, rp_g, ci_g, rows)
    alpha = x.alpha.double().numpy()
    ref_o = {r: O.combine(ref_s[r], ref_l[r], alpha[r[1]]) for r in rows}
    got = dict(o=U.rows_of(o, rows, wl.bq), s=U.rows_of(os_, rows, wl.bq), l=U.rows_of(ol, rows, wl.bq))
    return got, dict(o=ref_o, s=ref_s, l=ref_l), (rp_g, ci_g)


def test_tiny_fp32_workload_alpha_1_and_half():
    wl = gen.WORKLOADS["tiny-fp32-N1024"]
    for alpha in (1.0, 0.5):
        print(f"[attn] {wl.name} alpha={alpha}", flush=True)
        x = gen.make(wl.with_(alpha=(alpha,) * wl.H))
        got, ref, _ = _run_all(x)
        for key in ("o", "s", "l"):
            m, r = U.compare_rows(got[key], ref[key])
            print(f"  {key}: max-abs {m:.3g} rel {r:.3g}")
            _bar("fp32", m, r, key)


SMALL = [
    ("fp32-ragged-1000", "fp32", 1000, 64, 64, 64, 0.1, 0.6),
    ("fp32-ragged-1001-d128", "fp32", 1001, 128, 128, 64, 0.1, 0.5),
    ("bf16-ragged-1000", "bf16", 1000, 128, 128, 64, 0.1, 0.6),
    ("bf16-ragged-1001", "bf16", 1001, 128, 128, 64, 0.1, 0.6),
    ("bf16-d64", "bf16", 777, 64, 64, 64, 0.1, 0.6),
    ("bf16-bk128", "bf16", 1500, 128, 128, 128, 0.1, 0.6),
    ("bf16-bq64", "bf16", 1300, 128, 64, 64, 0.1, 0.6),
    ("bf16-d64-bq128-bk128", "bf16", 1100, 64, 128, 128, 0.2, 0.6),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small(case):
    name, dtype, N, d, bq, bk, k_frac, p = case
    print(f"[attn] {name}", flush=True)
    x = _adhoc(dtype, N, d, bq, bk, k_frac, p)
    got, ref, _ = _run_all(x)
    for key in ("o", "s", "l"):
        m, r = U.compare_rows(got[key], ref[key])
        print(f"  {key}: max-abs {m:.3g} rel {r:.3g}")
        _bar(dtype, m, r, f"{name}/{key}")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_empty_mask_is_linear_attention(dtype):
    """k_frac = p = 0: nothing selected, O_s = 0 and alpha = 0 gives linear
    attention over every key."""
    print(f"[attn] empty mask {dtype}", flush=True)
    x = _adhoc(dtype, 900, 128, 128, 64, 0.0, 0.0, alpha=(0.0, 0.0, 0.0))
    got, ref, (rp, ci) = _run_all(x)
    assert rp[-1] == 0
    assert all(np.all(v == 0) for v in got["s"].values())
    m, r = U.compare_rows(got["o"], ref["o"])
    _bar(dtype, m, r, "empty/o")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_full_mask_is_dense_attention(dtype):
    """k_frac = 1: every block selected, O_l = 0, and alpha = 1 is dense."""
    print(f"[attn] full mask {dtype}", flush=True)
    x = _adhoc(dtype, 700, 128, 128, 64, 1.0, 0.5, alpha=(1.0, 1.0, 1.0))
    got, ref, (rp, ci) = _run_all(x)
    assert all(np.all(v == 0) for v in got["l"].values())
    q, k, v = U.dev(x.Q, x.K, x.V)
    dn = S.sla_dense_fwd(q, k, v, 128, 64)
    rows = list(ref["o"].keys())
    dref = O.dense(x.Q, x.K, x.V, rows, bq=128)
    for name, g in (("attn", got["o"]), ("dense", U.rows_of(dn, rows, 128))):
        m, r = U.compare_rows(g, dref)
        _bar(dtype, m, r, f"full/{name}")


def _full_size(name, n_rows=32, x=None, **over):
    """Full-size parity on at least n_rows row blocks chosen from the GPU's
    mask (longest and shortest rows, partial last blocks, the ends of every
    XCD's row range, random rows); O, O_s and O_l each to the bf16 bar."""
    wl = gen.WORKLOADS[name].with_(**over) if over else gen.WORKLOADS[name]
    print(f"[attn] {wl.name} {over}", flush=True)
    x = gen.make(wl) if x is None else x
    pick = lambda rp: U.pick_rows(rp, wl.B, wl.H, wl.Nq, n=n_rows, seed=1)
    got, ref, (rp, ci) = _run_all(x, pick)
    counts = np.diff(rp)
    print(f"  rows {len(ref['o'])}, listed blocks per row {counts.min()}..{counts.max()}")
    for key in ("o", "s", "l"):
        if key == "l" and float(x.alpha.min()) == 1.0:
            continue
        m, r = U.compare_rows(got[key], ref[key])
        print(f"  {key}: max-abs {m:.3g} rel {r:.3g}")
        _bar("bf16", m, r, f"{wl.name}/{key}")


def test_480p_sparse_only():
    _full_size("video480p-sparse-N32760")


def test_480p_sla2():
    _full_size("video480p-sla2-N32760")


def test_720p_sla2():
    _full_size("video720p-sla2-N75600")


SWEEP = [(t, p) for t in gen.ROUTER_TAUS for p in gen.ROUTER_PS]


@pytest.mark.parametrize("tau,p", SWEEP, ids=[f"tau{t}-p{p}" for t, p in SWEEP])
def test_480p_router(tau, p):
    x = U.router_inputs(tau)
    x = dataclasses.replace(x, wl=x.wl.with_(p=p))
    _full_size("video480p-router-N32760", x=x, tau=tau, p=p)


def test_dense_480p_sampled():
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print("[attn] dense 480p", flush=True)
    x = gen.make(wl, heads=2)
    q, k, v = U.dev(x.Q, x.K, x.V)
    o = S.sla_dense_fwd(q, k, v, wl.bq, wl.bk)
    torch.cuda.synchronize()
    rows = U.sample_rows(1, 2, wl.Nq, 4, seed=3)
    m, r = U.compare_rows(U.rows_of(o, rows, wl.bq), O.dense(x.Q, x.K, x.V, rows, bq=wl.bq))
    print(f"  dense: max-abs {m:.3g} rel {r:.3g}")
    _bar("bf16", m, r, "dense")


def test_every_element_written_and_deterministic():
    """Outputs prefilled with NaN come back finite everywhere; two runs are
    bitwise identical."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    print("[attn] NaN sentinel + determinism", flush=True)
    x = gen.make(wl, heads=3)
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    outs = []
    for _ in range(2):
        o = torch.full_like(q, float("nan"))
        S.sla_attn_fwd(q, k, v, a, wl.bq, wl.bk, wl.k_frac, wl.p, out=o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
