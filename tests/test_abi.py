"""The C interface loads without a GPU, exports every declared symbol, and
rejects invalid arguments on the host before launching anything (CPU only:
no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import block_sparse_linear_sla_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")

pytestmark = pytest.mark.skipif(not os.path.exists(S.LIB_PATH),
                                reason="libsla.so not built (run __graft_entry__.build())")

INVALID, UNSUPPORTED, WORKSPACE, CAPACITY = -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(sla_[a-z_0-9]+)\s*\(", text, re.M)))


def test_exports_match_header():
    names = declared_functions()
    assert set(names) == set(S.EXPORTS), names
    L = S.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = S.lib()
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert len(L.sla_status_string(code)) > 0


def prob(**kw):
    base = dict(B=1, H=2, N=1024, d=64, bq=64, bk=64, dtype=S.SLA_F32)
    base.update(kw)
    return S.Problem(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(H=-1), INVALID), (dict(N=0), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(bq=32), UNSUPPORTED),
    (dict(bk=256), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(N=4096 * 64 + 1, bk=64, H=1), UNSUPPORTED),          # Nk > 4096
    (dict(B=64, H=64, N=8192, d=128), UNSUPPORTED),           # > 2^31 elements
])
def test_bad_problem(kw, code):
    L = S.lib()
    p = prob(**kw)
    sel = S.Select(0.1, 0.6, None, None)
    assert L.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(sel)) == 0
    assert L.sla_mask_capacity(ctypes.byref(p)) == -1
    st = None
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, 1 << 30, None,
                      FAKE, 1 << 40, st) == code
    assert L.sla_sparse_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, st) == code
    assert L.sla_linear_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, st) == code
    assert L.sla_attn_fwd(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          1 << 30, FAKE, 1 << 40, st) == code
    assert L.sla_dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, st) == code
    assert L.sla_kv_prepare(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1 << 40, st) == code
    assert L.sla_fused_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                           st) == code


def test_null_problem_and_select():
    L = S.lib()
    p = prob()
    assert L.sla_workspace_bytes(None, None) == 0
    assert L.sla_mask(None, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, FAKE, 1 << 40, None) == INVALID
    assert L.sla_mask(ctypes.byref(p), None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None, FAKE, 1 << 40,
                      None) == INVALID


@pytest.mark.parametrize("kf,pp", [(-0.1, 0.5), (1.5, 0.5), (0.1, -1e-3), (0.1, 1.01),
                                   (float("nan"), 0.5), (0.1, float("nan"))])
def test_bad_selection_parameters(kf, pp):
    L = S.lib()
    p = prob()
    sel = S.Select(kf, pp, None, None)
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, 1 << 30, None, FAKE,
                      1 << 40, None) == INVALID
    assert L.sla_attn_fwd(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          1 << 30, FAKE, 1 << 40, None) == INVALID


def test_router_needs_both_matrices():
    L = S.lib()
    p = prob()
    sel = S.Select(0.1, 0.6, FAKE, None)
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, 1 << 30, None, FAKE,
                      1 << 40, None) == INVALID


def test_null_tensors():
    L = S.lib()
    p = prob()
    sel = S.Select(0.1, 0.6, None, None)
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), None, FAKE, FAKE, FAKE, 1 << 30, None, FAKE,
                      1 << 40, None) == INVALID
    assert L.sla_sparse_fwd(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == INVALID
    assert L.sla_sparse_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == INVALID
    assert L.sla_linear_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None) == INVALID
    assert L.sla_attn_fwd(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                          1 << 30, FAKE, 1 << 40, None) == INVALID    # alpha
    assert L.sla_dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, None) == INVALID
    assert L.sla_kv_prepare(ctypes.byref(p), None, FAKE, None, FAKE, 1 << 40, None) == INVALID
    assert L.sla_fused_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                           None) == INVALID   # alpha


def test_capacity_and_workspace_checks():
    L = S.lib()
    p = prob()
    sel = S.Select(0.1, 0.6, None, None)
    cap = L.sla_mask_capacity(ctypes.byref(p))
    assert cap == 1 * 2 * 16 * 16
    need = L.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(sel))
    assert need > 0
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, cap - 1, None, FAKE,
                      need, None) == CAPACITY
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, cap, None, FAKE,
                      need - 1, None) == WORKSPACE
    assert L.sla_mask(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, cap, None, None,
                      need, None) == WORKSPACE
    assert L.sla_linear_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == WORKSPACE
    assert L.sla_attn_fwd(ctypes.byref(p), ctypes.byref(sel), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          cap - 1, FAKE, need, None) == CAPACITY
    assert L.sla_kv_prepare(ctypes.byref(p), FAKE, FAKE, None, FAKE, 16, None) == WORKSPACE
    assert L.sla_fused_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                           None) == WORKSPACE


def test_workspace_grows_with_router():
    L = S.lib()
    p = prob(B=2, H=16, N=32760, d=128, bq=128, bk=64, dtype=S.SLA_BF16)
    a = L.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(S.Select(0.03, 0.6, None, None)))
    b = L.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(S.Select(0.03, 0.6, FAKE, FAKE)))
    assert b > a > 0


@pytest.mark.parametrize("T", [0.0, -1.0, float("nan"), float("inf")])
def test_soft_topk_temperature(T):
    L = S.lib()
    p = prob()
    sel = S.Select(0.1, 0.0, None, None)
    assert L.sla_soft_topk(ctypes.byref(p), ctypes.byref(sel), T, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                           None) == INVALID


def test_soft_topk_null_and_workspace():
    L = S.lib()
    p = prob()
    sel = S.Select(0.1, 0.0, None, None)
    assert L.sla_soft_topk(ctypes.byref(p), ctypes.byref(sel), 0.5, None, FAKE, FAKE, FAKE, 1 << 40,
                           None) == INVALID
    assert L.sla_soft_topk(ctypes.byref(p), ctypes.byref(sel), 0.5, FAKE, FAKE, None, FAKE, 1 << 40,
                           None) == INVALID
    assert L.sla_soft_topk(ctypes.byref(p), ctypes.byref(sel), 0.5, FAKE, FAKE, FAKE, FAKE, 16,
                           None) == WORKSPACE
    bad = S.Select(1.5, 0.0, None, None)
    assert L.sla_soft_topk(ctypes.byref(p), ctypes.byref(bad), 0.5, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                           None) == INVALID


def test_i8_layout_and_limits():
    L = S.lib()
    p = prob(N=1000, d=128, bq=128, bk=64, dtype=S.SLA_BF16)
    lay = S.I8Layout()
    assert L.sla_i8_layout_of(ctypes.byref(p), ctypes.byref(lay)) == 0
    BH, Nq, Nk = 2, 8, 16
    sizes = [("q8", BH * Nq * 128 * 128), ("k8", BH * Nk * 64 * 128), ("vt8", BH * Nk * 64 * 128),
             ("sq", BH * Nq * 4), ("sk", BH * Nk * 4), ("sv", BH * 128 * 4), ("rv", BH * 128 * 4),
             ("vpart", BH * 1 * 128 * 4)]
    off = 0
    for name, n in sizes:  # regions in order, each 256-byte aligned, no overlap
        assert getattr(lay, name) == off, name
        off = (off + n + 255) // 256 * 256
    assert lay.total == off
    assert L.sla_i8_layout_of(ctypes.byref(p), None) == INVALID
    big = prob(N=131073, H=1, d=64, bk=128)
    assert L.sla_i8_layout_of(ctypes.byref(big), ctypes.byref(lay)) == UNSUPPORTED
    for fmt in ("i8", "i8f8"):
        quant, fwd = getattr(L, "sla_quantize_" + fmt), getattr(L, "sla_sparse_fwd_" + fmt)
        assert quant(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED
        assert fwd(ctypes.byref(big), FAKE, 1 << 40, FAKE, FAKE, FAKE, None) == UNSUPPORTED
        bad = prob(d=96)
        assert quant(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED


@pytest.mark.parametrize("fmt", ["i8", "i8f8"])
def test_8bit_null_and_buffer_checks(fmt):
    L = S.lib()
    quant, fwd = getattr(L, "sla_quantize_" + fmt), getattr(L, "sla_sparse_fwd_" + fmt)
    p = prob(dtype=S.SLA_BF16)
    lay = S.I8Layout()
    assert L.sla_i8_layout_of(ctypes.byref(p), ctypes.byref(lay)) == 0
    n = lay.total
    for args in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        assert quant(ctypes.byref(p), *args, FAKE, n, None) == INVALID
    assert quant(ctypes.byref(p), FAKE, FAKE, FAKE, None, n, None) == WORKSPACE
    assert quant(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, n - 1, None) == WORKSPACE
    for args in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        assert fwd(ctypes.byref(p), FAKE, n, *args, None) == INVALID
    assert fwd(ctypes.byref(p), None, n, FAKE, FAKE, FAKE, None) == WORKSPACE
    assert fwd(ctypes.byref(p), FAKE, n - 1, FAKE, FAKE, FAKE, None) == WORKSPACE
    assert fwd(None, FAKE, n, FAKE, FAKE, FAKE, None) == INVALID


def test_bwd_checks():
    L = S.lib()
    p32 = prob()
    p16 = prob(dtype=S.SLA_BF16)
    n = L.sla_bwd_workspace_bytes(ctypes.byref(p16))
    assert n > 0 and L.sla_bwd_workspace_bytes(None) == 0
    args = [FAKE] * 9
    assert L.sla_sparse_bwd(ctypes.byref(p32), *args, FAKE, n, None) == UNSUPPORTED
    for i in range(9):
        a = list(args)
        a[i] = None
        assert L.sla_sparse_bwd(ctypes.byref(p16), *a, FAKE, n, None) == INVALID, i
    assert L.sla_sparse_bwd(ctypes.byref(p16), *args, None, n, None) == WORKSPACE
    assert L.sla_sparse_bwd(ctypes.byref(p16), *args, FAKE, n - 1, None) == WORKSPACE
    for i in range(4):
        a = [FAKE] * 4
        a[i] = None
        assert L.sla_alpha_grad(ctypes.byref(p32), *a, FAKE, n, None) == INVALID, i
    assert L.sla_alpha_grad(ctypes.byref(p16), FAKE, FAKE, FAKE, FAKE, FAKE, n - 1, None) == WORKSPACE


def test_linear_and_mixed_bwd_checks():
    L = S.lib()
    p32 = prob()
    p16 = prob(dtype=S.SLA_BF16)
    n = L.sla_bwd_workspace_bytes(ctypes.byref(p16))
    lin = [FAKE] * 9
    assert L.sla_linear_bwd(ctypes.byref(p32), *lin, 0, FAKE, n, None) == UNSUPPORTED
    for i in range(9):
        a = list(lin)
        a[i] = None
        assert L.sla_linear_bwd(ctypes.byref(p16), *a, 1, FAKE, n, None) == INVALID, i
    assert L.sla_linear_bwd(ctypes.byref(p16), *lin, 0, None, n, None) == WORKSPACE
    assert L.sla_linear_bwd(ctypes.byref(p16), *lin, 0, FAKE, n - 1, None) == WORKSPACE
    assert L.sla_linear_bwd(None, *lin, 0, FAKE, n, None) == INVALID
    mixed = [FAKE] * 10  # Q, K, V, dO, alpha, row_ptr, col_idx, dQ, dK, dV
    assert L.sla_attn_bwd(ctypes.byref(p32), *mixed, None, FAKE, n, None) == UNSUPPORTED
    for i in range(10):
        a = list(mixed)
        a[i] = None
        assert L.sla_attn_bwd(ctypes.byref(p16), *a, FAKE, FAKE, n, None) == INVALID, i
    assert L.sla_attn_bwd(ctypes.byref(p16), *mixed, FAKE, None, n, None) == WORKSPACE
    assert L.sla_attn_bwd(ctypes.byref(p16), *mixed, None, FAKE, n - 1, None) == WORKSPACE


def test_saved_pair_checks():
    """sla_fused_fwd_save and sla_attn_bwd_saved: bf16 only, every pointer
    required, the workspaces checked; the saved-terms count is B*H*Nq*bq."""
    L = S.lib()
    p32 = prob()
    p16 = prob(dtype=S.SLA_BF16, N=1000, bq=128)
    assert L.sla_saved_terms_count(ctypes.byref(p16)) == 2 * 8 * 128
    assert L.sla_saved_terms_count(ctypes.byref(prob(B=0))) == -1
    sel = S.select(0.1, 0.5)
    nf = L.sla_workspace_bytes(ctypes.byref(p16), ctypes.byref(sel))
    fwd = [FAKE] * 7  # Q, K, V, alpha, row_ptr, col_idx, O
    sv = [FAKE] * 4   # lse2, invden, O_s, O_l
    assert L.sla_fused_fwd_save(ctypes.byref(p32), *fwd, FAKE, nf, *sv, None) == UNSUPPORTED
    for i in range(11):
        a = fwd + sv
        a[i] = None
        assert L.sla_fused_fwd_save(ctypes.byref(p16), *a[:7], FAKE, nf, *a[7:], None) == INVALID, i
    assert L.sla_fused_fwd_save(ctypes.byref(p16), *fwd, None, nf, *sv, None) == WORKSPACE
    assert L.sla_fused_fwd_save(ctypes.byref(p16), *fwd, FAKE, nf - 1, *sv, None) == WORKSPACE
    nb = L.sla_bwd_workspace_bytes(ctypes.byref(p16))
    bwd = [FAKE] * 14  # Q, K, V, dO, alpha, row_ptr, col_idx, lse2, invden, O_s, O_l, dQ, dK, dV
    assert L.sla_attn_bwd_saved(ctypes.byref(p32), *bwd, None, FAKE, nb, None) == UNSUPPORTED
    for i in range(14):
        a = list(bwd)
        a[i] = None
        assert L.sla_attn_bwd_saved(ctypes.byref(p16), *a, FAKE, FAKE, nb, None) == INVALID, i
    assert L.sla_attn_bwd_saved(ctypes.byref(p16), *bwd, FAKE, None, nb, None) == WORKSPACE
    assert L.sla_attn_bwd_saved(ctypes.byref(p16), *bwd, None, FAKE, nb - 1, None) == WORKSPACE
    assert L.sla_attn_bwd_saved(None, *bwd, None, FAKE, nb, None) == INVALID


def test_mask_prepared_checks():
    L = S.lib()
    p = prob(dtype=S.SLA_BF16)
    sel = S.select(0.1, 0.5)
    n = L.sla_workspace_bytes(ctypes.byref(p), ctypes.byref(sel))
    cap = L.sla_mask_capacity(ctypes.byref(p))
    args = [FAKE] * 5  # Q, K, alpha, row_ptr, col_idx
    for i in range(5):
        a = list(args)
        a[i] = None
        assert L.sla_mask_prepared(ctypes.byref(p), ctypes.byref(sel), *a, cap, FAKE, n, None) == INVALID, i
    assert L.sla_mask_prepared(ctypes.byref(p), ctypes.byref(sel), *args, cap - 1, FAKE, n, None) == CAPACITY
    assert L.sla_mask_prepared(ctypes.byref(p), ctypes.byref(sel), *args, cap, None, n, None) == WORKSPACE
    assert L.sla_mask_prepared(ctypes.byref(p), ctypes.byref(sel), *args, cap, FAKE, n - 1, None) == WORKSPACE
    assert L.sla_mask_prepared(None, ctypes.byref(sel), *args, cap, FAKE, n, None) == INVALID
    assert L.sla_mask_prepared(ctypes.byref(p), None, *args, cap, FAKE, n, None) == INVALID


def test_binding_refuses_host_tensors_and_wrong_saved_dtypes():
    """The Python binding checks its tensors before any call reaches the
    library: host tensors, and saved branch outputs that are not float32."""
    import torch
    q = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.sla_sparse_fwd(q, q, q, 64, 64, None, None)
    saved = dict(lse2=torch.zeros(8), invden=torch.zeros(8), o_s=q, o_l=q)
    with pytest.raises(ValueError):
        S.sla_attn_bwd_saved(q, q, q, q, torch.zeros(2), 64, 64, None, None, saved)
