"""The library's calls under HIP graph capture.

Every library call only launches kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a whole forward step or a
whole backward call can be captured once and replayed.  Each test captures
into static buffers, then for several input sets in a row: copies the set
into the static inputs, replays, and runs the same calls eagerly into
separate buffers; the replay must equal the eager result bit for bit (the
kernels sum in fixed orders), every time."""
import pytest
import torch

import block_sparse_linear_sla_amd as S
import gen
from tests import _util as U

pytestmark = pytest.mark.gpu


def _step(q, k, v, a, wl, ws, rp, ci, out):
    S.sla_kv_prepare(k, v, wl.bq, wl.bk, ws, a)
    S.sla_mask_prepared(q, k, a, wl.bq, wl.bk, wl.k_frac, wl.p, ws=ws, row_ptr=rp, col_idx=ci)
    S.sla_fused_fwd(q, k, v, a, wl.bq, wl.bk, rp, ci, ws, out=out)


def _buffers(q, wl, cap):
    dev = q.device
    prob, sel = S.problem(q, wl.bq, wl.bk), S.select(wl.k_frac, wl.p)
    ws = S.workspace(prob, sel, dev)
    rp = torch.empty(wl.B * q.shape[1] * wl.Nq + 1, dtype=torch.int32, device=dev)
    ci = torch.full((cap,), -1, dtype=torch.int32, device=dev)
    return ws, rp, ci, torch.empty_like(q)


def test_forward_step_graph_replays():
    """sla_kv_prepare + sla_mask_prepared + sla_fused_fwd (the forward step)
    captured on the 480p SLA2 workload (three heads), replayed on three input
    sets."""
    wl = gen.WORKLOADS["video480p-sla2-N32760"]
    sets = [U.dev(x.Q, x.K, x.V, x.alpha) for x in (gen.make(wl, seed=s, heads=3) for s in (41, 42, 43))]
    q, k, v, a = (t.clone() for t in sets[0])
    cap = S.sla_mask_capacity(S.problem(q, wl.bq, wl.bk))
    ws, rp, ci, out = _buffers(q, wl, cap)
    _step(q, k, v, a, wl, ws, rp, ci, out)  # eager run before the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("[graph] capturing the forward step", flush=True)
    with torch.cuda.graph(g):
        _step(q, k, v, a, wl, ws, rp, ci, out)
    torch.cuda.synchronize()
    ews, erp, eci, eout = _buffers(q, wl, cap)
    for n, src in enumerate(sets + sets[:1]):
        for dst, t in zip((q, k, v, a), src):
            dst.copy_(t)
        g.replay()
        torch.cuda.synchronize()
        _step(q, k, v, a, wl, ews, erp, eci, eout)
        torch.cuda.synchronize()
        nnz = int(rp[-1])
        print(f"  replay {n}: nnz {nnz}", flush=True)
        assert torch.equal(rp, erp), f"replay {n}: row_ptr differs"
        assert torch.equal(ci[:nnz], eci[:nnz]), f"replay {n}: col_idx differs"
        assert torch.equal(out.view(torch.int16), eout.view(torch.int16)), f"replay {n}: output differs"
        if n == 0:
            first = out.clone()
        elif n < len(sets):
            assert not torch.equal(out, first), "the replay did not see the new inputs"
        else:  # the first set again
            assert torch.equal(out.view(torch.int16), first.view(torch.int16)), "set 0 replayed differently"


def test_backward_graph_replays():
    """sla_attn_bwd (mask transpose, both branches' gradients) captured on a
    ragged shape with the library's mask, replayed on three output
    gradients."""
    wl = gen.Workload("adhoc", B=1, H=3, grid=(1, 1, 5001), d=128, bq=128, bk=64, k_frac=0.1, p=0.7,
                      dtype="bf16", router=False, seed=29)
    x = gen.make(wl)
    q, k, v, a = U.dev(x.Q, x.K, x.V, x.alpha)
    rp, ci = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    gens = [torch.Generator().manual_seed(s) for s in (1, 2, 3)]
    dos = [torch.randn(tuple(q.shape), generator=gg).to(torch.bfloat16).cuda() for gg in gens]
    do = dos[0].clone()
    prob = S.problem(q, wl.bq, wl.bk)
    ws, ews = S.bwd_workspace(prob, q.device), S.bwd_workspace(prob, q.device)
    grads = tuple(torch.empty_like(q) for _ in range(3))
    egrads = tuple(torch.empty_like(q) for _ in range(3))
    S.sla_attn_bwd(q, k, v, do, a, wl.bq, wl.bk, rp, ci, ws=ws, out=grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("[graph] capturing sla_attn_bwd", flush=True)
    with torch.cuda.graph(g):
        S.sla_attn_bwd(q, k, v, do, a, wl.bq, wl.bk, rp, ci, ws=ws, out=grads)
    torch.cuda.synchronize()
    for n, src in enumerate(dos + dos[:1]):
        do.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        S.sla_attn_bwd(q, k, v, do, a, wl.bq, wl.bk, rp, ci, ws=ews, out=egrads)
        torch.cuda.synchronize()
        print(f"  replay {n}", flush=True)
        for name, t, e in zip(("dQ", "dK", "dV"), grads, egrads):
            assert torch.equal(t.view(torch.int16), e.view(torch.int16)), f"replay {n}: {name} differs"


def test_training_pair_graph_replays():
    """sla_fused_fwd_save followed by sla_attn_bwd_saved (with the alpha
    gradient) captured as one graph on a ragged shape with the library's
    mask, replayed on three input sets; every output of every replay equals
    the eager calls' bit for bit."""
    wl = gen.Workload("adhoc", B=1, H=3, grid=(1, 1, 5001), d=128, bq=128, bk=64, k_frac=0.1, p=0.7,
                      dtype="bf16", router=False, seed=29)
    sets = []
    for s in (5, 6, 7):
        x = gen.make(wl, seed=s)
        g = torch.Generator().manual_seed(s)
        sets.append(U.dev(x.Q, x.K, x.V, x.alpha) + (torch.randn(tuple(x.Q.shape), generator=g).to(torch.bfloat16).cuda(),))
    q, k, v, a, do = (t.clone() for t in sets[0])
    rp, ci = S.sla_mask(q, k, wl.bq, wl.bk, wl.k_frac, wl.p)
    prob, sel = S.problem(q, wl.bq, wl.bk), S.select(wl.k_frac, wl.p)

    def buffers():
        ws = S.workspace(prob, sel, q.device)
        _, sv = S.sla_fused_fwd_save(q, k, v, a, wl.bq, wl.bk, rp, ci, ws)  # allocates the saved terms
        return dict(ws=ws, bws=S.bwd_workspace(prob, q.device), o=torch.empty_like(q), sv=sv,
                    grads=tuple(torch.empty_like(q) for _ in range(3)),
                    da=torch.empty(q.shape[1], dtype=torch.float32, device=q.device))

    def run(b):
        S.sla_kv_prepare(k, v, wl.bq, wl.bk, b["ws"], a)
        S.sla_fused_fwd_save(q, k, v, a, wl.bq, wl.bk, rp, ci, b["ws"], out=b["o"], saved=b["sv"])
        S.sla_attn_bwd_saved(q, k, v, do, a, wl.bq, wl.bk, rp, ci, b["sv"], ws=b["bws"], out=b["grads"],
                             dalpha=b["da"])

    st, eg = buffers(), buffers()
    run(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("[graph] capturing the training pair", flush=True)
    with torch.cuda.graph(g):
        run(st)
    torch.cuda.synchronize()
    for n, src in enumerate(sets):
        for dst, t in zip((q, k, v, a, do), src):
            dst.copy_(t)
        g.replay()
        torch.cuda.synchronize()
        run(eg)
        torch.cuda.synchronize()
        print(f"  replay {n}", flush=True)
        pairs = [("O", st["o"], eg["o"]), ("dalpha", st["da"], eg["da"])]
        pairs += [(key, st["sv"][key], eg["sv"][key]) for key in ("lse2", "invden", "o_s", "o_l")]
        pairs += [(name, t, e) for name, t, e in zip(("dQ", "dK", "dV"), st["grads"], eg["grads"])]
        for name, t, e in pairs:
            assert torch.equal(t, e), f"replay {n}: {name} differs"
