"""GPU parity of sla_mask against the oracle: the CSR must match exactly except
at blocks that sit on the selection cut (pooled logit within 1e-5 of the
threshold logit, or cumulative mass within 1e-5 of p); the float64 pooled
logits must agree to float64 rounding."""
import numpy as np
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from oracle import sla_oracle as O
from tests import _util as U

pytestmark = pytest.mark.gpu

SMALL = [
    # name, dtype, N, d, bq, bk, k_frac, p, router
    ("fp32-ragged-1000", "fp32", 1000, 64, 64, 64, 0.1, 0.6, False),
    ("fp32-ragged-1001-d128", "fp32", 1001, 128, 128, 64, 0.1, 0.6, False),
    ("bf16-ragged-1000", "bf16", 1000, 128, 128, 64, 0.05, 0.9, False),
    ("bf16-ragged-1001-d64", "bf16", 1001, 64, 64, 128, 0.2, 0.5, False),
    ("bf16-bq128-bk128", "bf16", 4000, 128, 128, 128, 0.1, 0.7, False),
    ("bf16-router", "bf16", 2000, 128, 128, 64, 0.03, 0.6, True),
    ("bf16-empty", "bf16", 1500, 128, 128, 64, 0.0, 0.0, False),
    ("bf16-topk-only", "bf16", 1500, 128, 128, 64, 0.25, 0.0, False),
    ("bf16-full", "bf16", 700, 128, 128, 64, 1.0, 0.5, False),
    ("bf16-p1", "bf16", 1500, 128, 128, 64, 0.0, 1.0, False),
    # a long kept prefix (about 77 of 128 blocks per row): both cuts deep in
    # the row
    ("bf16-long-prefix", "bf16", 8192, 128, 128, 64, 0.6, 0.5, False),
    # Top-p decides the count (k = 1)
    ("bf16-p-dominant", "bf16", 3000, 128, 128, 64, 0.02, 0.95, False),
    # blocks per lane that are not powers of two: Nk = 625 (12 per lane) and
    # Nk = 1400 (24 per lane)
    ("bf16-Nk625", "bf16", 40000, 128, 128, 64, 0.05, 0.7, False),
    ("bf16-Nk1400", "bf16", 89600, 64, 128, 64, 0.03, 0.6, False),
]


def _small_inputs(dtype, N, d, bq, bk, k_frac, p, router, seed=7):
    wl = gen.Workload("adhoc", B=2, H=3, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=k_frac, p=p,
                      dtype=dtype, router=router, seed=seed)
    return gen.make(wl)


def run_and_check(x, k_frac, p, check_logits=True):
    wl = x.wl
    q, k = U.dev(x.Q, x.K)
    wq, wk = U.dev(x.Wq, x.Wk)
    rp, ci, logits = S.sla_mask(q, k, wl.bq, wl.bk, k_frac, p, wq, wk, return_logits=True)
    torch.cuda.synchronize()
    rp_g, ci_g = U.csr(rp, ci)
    rp_o, ci_o, meta = U.oracle_mask_per_head(x, k_frac, p)
    B, H, N, _ = x.Q.shape
    Nq, Nk = O.n_blocks(N, wl.bq), O.n_blocks(N, wl.bk)
    U.check_csr_structure(rp_g, ci_g, B * H * Nq, Nk)
    if check_logits:
        Sg = logits.cpu().numpy().reshape(meta["S"].shape)
        err = np.max(np.abs(Sg - meta["S"]) / np.maximum(1.0, np.abs(meta["S"])))
        assert err < 1e-10, f"pooled logits differ by {err}"
    bad, excused, rows = U.mask_mismatches(rp_g, ci_g, rp_o, ci_o, meta, p)
    assert not bad, f"{len(bad)} unexcused mask differences, e.g. {bad[:5]}"
    return rp_g, ci_g, excused, rows


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_mask_small(case):
    name, dtype, N, d, bq, bk, k_frac, p, router = case
    print(f"[mask] {name}", flush=True)
    x = _small_inputs(dtype, N, d, bq, bk, k_frac, p, router)
    rp, ci, excused, rows = run_and_check(x, k_frac, p)
    Nk = O.n_blocks(N, bk)
    R = len(rp) - 1
    if k_frac == 0 and p == 0:
        assert rp[-1] == 0
    if k_frac == 1:
        assert rp[-1] == R * Nk


def test_mask_tiny_workload():
    wl = gen.WORKLOADS["tiny-fp32-N1024"]
    print(f"[mask] {wl.name}", flush=True)
    x = gen.make(wl)
    rp, ci, excused, rows = run_and_check(x, wl.k_frac, wl.p)
    assert rows == 0  # nothing near the cut at this size


@pytest.mark.parametrize("name", ["video480p-sparse-N32760", "video480p-sla2-N32760"])
def test_mask_480p(name):
    wl = gen.WORKLOADS[name]
    print(f"[mask] {name}", flush=True)
    x = gen.make(wl)
    rp, ci, excused, rows = run_and_check(x, wl.k_frac, wl.p)
    sparsity = 1 - rp[-1] / float(wl.B * wl.H * wl.Nq * wl.Nk)
    print(f"  sparsity {sparsity:.4f}, differing rows {rows}, excused blocks {excused}")


SWEEP = [(t, p) for t in gen.ROUTER_TAUS for p in gen.ROUTER_PS]


@pytest.mark.parametrize("tau,p", SWEEP, ids=[f"tau{t}-p{p}" for t, p in SWEEP])
def test_mask_router_sweep(tau, p):
    """Every point of the distribution sweep: flat pooled maps (tau = 0.25,
    where Top-p keeps up to about half of the blocks) to peaked ones (tau = 4)."""
    x = U.router_inputs(tau)
    wl = x.wl.with_(p=p)
    print(f"[mask] router tau={tau} p={p}", flush=True)
    rp, ci, excused, rows = run_and_check(x, wl.k_frac, p)
    counts = np.diff(rp)
    print(f"  sparsity {1 - rp[-1] / float(wl.B * wl.H * wl.Nq * wl.Nk):.4f}, blocks per row "
          f"{counts.min()}..{counts.max()}, excused {excused}")


def test_mask_720p():
    wl = gen.WORKLOADS["video720p-sla2-N75600"]
    print(f"[mask] {wl.name}", flush=True)
    x = gen.make(wl)
    rp, ci, excused, rows = run_and_check(x, wl.k_frac, wl.p, check_logits=True)
    print(f"  sparsity {1 - rp[-1] / float(wl.B * wl.H * wl.Nq * wl.Nk):.4f}, excused {excused}")


TIES = [
    # name, dtype, N, d, bq, bk, k_frac, p (N a multiple of bk: every key block full)
    ("fp32-ties-Nk16", "fp32", 1024, 64, 64, 64, 0.1, 0.5),
    ("bf16-ties-Nk512", "bf16", 32768, 128, 128, 64, 0.03, 0.5),
    ("bf16-ties-Nk512-p0.2", "bf16", 32768, 128, 128, 64, 0.03, 0.2),
]


@pytest.mark.parametrize("case", TIES, ids=[c[0] for c in TIES])
def test_mask_exact_ties(case):
    """Exactly tied pooled keys, decided by the lower block index on both sides,
    so the CSR must equal the oracle's with nothing excused.  Head 0 has Q = 0:
    every logit is 0 and P = 1/Nk exactly (Nk a power of two, so every partial
    sum is exact), so every row keeps blocks 0 .. max(ceil(k_frac Nk),
    ceil(p Nk)) - 1 (256 blocks at Nk = 512 and p = 0.5: the Top-p cut
    falls inside one tie of all Nk blocks, which no bisection on the logit
    can split).  Head 1 repeats key blocks 0..3 over the row
    (four groups of equal P, the cut inside the top group); head 2 is the
    random control."""
    name, dtype, N, d, bq, bk, k_frac, p = case
    print(f"[mask] {name}", flush=True)
    x = _small_inputs(dtype, N, d, bq, bk, k_frac, p, False)
    B, H = x.Q.shape[:2]
    Nq, Nk = O.n_blocks(N, bq), O.n_blocks(N, bk)
    assert N == Nk * bk and Nk % 4 == 0
    x.Q[:, 0] = 0
    kb = x.K[:, 1].reshape(B, Nk, bk, d)
    x.K[:, 1] = kb[:, :4].repeat(1, Nk // 4, 1, 1).reshape(B, N, d)
    q, k = U.dev(x.Q, x.K)
    rp, ci = S.sla_mask(q, k, bq, bk, k_frac, p)
    torch.cuda.synchronize()
    rp_g, ci_g = U.csr(rp, ci)
    rp_o, ci_o, _ = U.oracle_mask_per_head(x, k_frac, p, keep_info=False)
    U.check_csr_structure(rp_g, ci_g, B * H * Nq, Nk)
    n0 = max(int(np.ceil(k_frac * Nk)), int(np.ceil(p * Nk - 1e-9)))
    for b in range(B):
        for i in range(Nq):
            r = (b * H + 0) * Nq + i
            assert np.array_equal(ci_g[rp_g[r]:rp_g[r + 1]], np.arange(n0)), f"head 0 row {r}"
    assert np.array_equal(rp_g, rp_o), "row counts differ from the oracle"
    assert np.array_equal(ci_g, ci_o), "column indices differ from the oracle"


def test_mask_deterministic():
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    x = gen.make(wl, heads=2)
    q, k = U.dev(x.Q, x.K)
    a = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    b = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    n = int(a[0][-1])
    assert torch.equal(a[0], b[0]) and torch.equal(a[1][:n], b[1][:n])


PREPARED = [
    # name, dtype, N, d, bq, bk, router, alpha per head (B=2, H=3)
    ("bf16-ragged-1000", "bf16", 1000, 128, 128, 64, False, (0.7, 1.0, 0.9)),
    ("bf16-ragged-1001-d64-bk128", "bf16", 1001, 64, 64, 128, False, (0.6, 0.8, 1.0)),
    ("bf16-router", "bf16", 2000, 128, 128, 64, True, (0.75, 0.6, 0.95)),
    ("bf16-bk128", "bf16", 4000, 128, 128, 128, False, (1.0, 1.0, 0.5)),
    ("fp32-ragged-1000", "fp32", 1000, 64, 64, 64, False, (0.5, 1.0, 0.7)),
]


@pytest.mark.parametrize("case", PREPARED, ids=[c[0] for c in PREPARED])
def test_mask_prepared_matches_mask(case):
    """sla_kv_prepare pools K for the heads it processes (alpha != 1, bf16);
    sla_mask_prepared then pools only the rest.  The CSR must be sla_mask's,
    entry for entry (the key-block means are float64 sums of bf16 values,
    exact in any order), and sla_attn_fwd, which runs the stages in that
    order, must give the output of the three separate calls; so must sla_mask
    (own workspace, on a second stream of the caller's) beside sla_kv_prepare,
    then sla_fused_fwd."""
    name, dtype, N, d, bq, bk, router, alpha = case
    print(f"[mask-prepared] {name}", flush=True)
    wl = gen.Workload("adhoc", B=2, H=3, grid=(1, 1, N), d=d, bq=bq, bk=bk, k_frac=0.1, p=0.6,
                      dtype=dtype, router=router, alpha=alpha, seed=17)
    x = gen.make(wl)
    q, k, v = U.dev(x.Q, x.K, x.V)
    wq, wk = U.dev(x.Wq, x.Wk)
    a = torch.tensor(alpha, dtype=torch.float32, device="cuda")
    prob, sel = S.problem(q, bq, bk), S.select(wl.k_frac, wl.p, wq, wk)
    ws = S.workspace(prob, sel, q.device)
    rp0, ci0 = S.sla_mask(q, k, bq, bk, wl.k_frac, wl.p, wq, wk)
    ws.fill_(0xFF)  # the prepared path must not rely on an earlier sla_mask in this workspace
    S.sla_kv_prepare(k, v, bq, bk, ws, a)
    rp1, ci1 = S.sla_mask_prepared(q, k, a, bq, bk, wl.k_frac, wl.p, wq, wk, ws=ws)
    torch.cuda.synchronize()
    n = int(rp0[-1])
    assert torch.equal(rp0, rp1) and torch.equal(ci0[:n], ci1[:n])
    o3 = S.sla_fused_fwd(q, k, v, a, bq, bk, rp1, ci1, ws)
    o1, rp2, ci2 = S.sla_attn_fwd(q, k, v, a, bq, bk, wl.k_frac, wl.p, wq, wk)
    torch.cuda.synchronize()
    assert torch.equal(rp0, rp2) and torch.equal(ci0[:n], ci2[:n])
    assert torch.equal(o1, o3)
    # the overlapped schedule spelled out with torch streams
    ws_m = S.workspace(prob, sel, q.device)
    rp4, ci4 = torch.full_like(rp1, -1), torch.full_like(ci1, -1)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    fork = torch.cuda.Event()
    fork.record(main)
    side.wait_event(fork)
    with torch.cuda.stream(side):
        S.sla_mask(q, k, bq, bk, wl.k_frac, wl.p, wq, wk, ws=ws_m, row_ptr=rp4, col_idx=ci4)
        join = torch.cuda.Event()
        join.record(side)
    ws2 = S.workspace(prob, sel, q.device)
    S.sla_kv_prepare(k, v, bq, bk, ws2, a)
    main.wait_event(join)
    o4 = S.sla_fused_fwd(q, k, v, a, bq, bk, rp4, ci4, ws2)
    torch.cuda.synchronize()
    assert torch.equal(rp0, rp4) and torch.equal(ci0[:n], ci4[:n])
    assert torch.equal(o1, o4)


def test_forward_calls_in_a_row_on_a_caller_stream():
    """Back-to-back sla_attn_fwd calls on a (non-default) stream of the
    caller's, on two inputs in turn with the same workspace and outputs, each
    give their own result: nothing of one call's work overlaps the next's."""
    wl = gen.Workload("adhoc", B=1, H=4, grid=(1, 1, 8192), d=128, bq=128, bk=64, k_frac=0.05, p=0.7,
                      dtype="bf16", alpha_range=(0.5, 0.9), seed=23)
    print("[attn-fwd] calls in a row on a caller stream", flush=True)
    xs = [gen.make(wl), gen.make(wl.with_(seed=24))]
    ins = [U.dev(x.Q, x.K, x.V, x.alpha) for x in xs]
    ref = []
    for q, k, v, a in ins:
        o, rp, ci = S.sla_attn_fwd(q, k, v, a, wl.bq, wl.bk, wl.k_frac, wl.p)
        torch.cuda.synchronize()
        ref.append((o.clone(), rp.clone()))
    assert not torch.equal(ref[0][0], ref[1][0])
    q0 = ins[0][0]
    prob, sel = S.problem(q0, wl.bq, wl.bk), S.select(wl.k_frac, wl.p)
    ws = S.workspace(prob, sel, q0.device)
    rp = torch.empty_like(ref[0][1])
    ci = torch.empty(S.sla_mask_capacity(prob), dtype=torch.int32, device=q0.device)
    out = torch.empty_like(q0)
    st = torch.cuda.Stream()
    got = []
    with torch.cuda.stream(st):
        for i in range(6):
            q, k, v, a = ins[i % 2]
            S.sla_attn_fwd(q, k, v, a, wl.bq, wl.bk, wl.k_frac, wl.p, out=out, ws=ws, row_ptr=rp, col_idx=ci)
            got.append((out.clone(), rp.clone()))
    st.synchronize()
    for i, (o, r) in enumerate(got):
        assert torch.equal(r, ref[i % 2][1]), f"call {i}: row_ptr"
        assert torch.equal(o, ref[i % 2][0]), f"call {i}: output"
