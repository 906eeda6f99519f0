"""Python binding of libsla.so, the gfx950 sparse + linear attention forward.

Argument marshalling only: every step of the computation runs in the HIP
library.  Tensors are torch CUDA tensors (device memory); work goes on
torch's current stream.  The functions carry the C interface's names
(include/sla.h); each allocates its outputs and workspace with torch unless
buffers are passed in.

There is no fallback: if libsla.so is missing or cannot be loaded, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SLA_LIB", os.path.join(_HERE, "libsla.so"))

SLA_F32, SLA_BF16 = 0, 1
STATUS = {0: "SLA_OK", -1: "SLA_ERR_INVALID_ARG", -2: "SLA_ERR_UNSUPPORTED",
          -3: "SLA_ERR_WORKSPACE", -4: "SLA_ERR_CAPACITY", -5: "SLA_ERR_HIP", -6: "SLA_ERR_TOO_LARGE"}
NOALLOC_SCRATCH_BYTES = 64 << 20
EXPORTS = ("sla_workspace_bytes", "sla_mask_capacity", "sla_mask", "sla_mask_prepared", "sla_soft_topk",
           "sla_mask_noalloc_bytes", "sla_mask_noalloc",
           "sla_sparse_fwd",
           "sla_linear_fwd", "sla_attn_fwd", "sla_kv_prepare", "sla_fused_fwd", "sla_saved_terms_count",
           "sla_fused_fwd_save",
           "sla_dense_fwd", "sla_i8_layout_of", "sla_quantize_i8", "sla_sparse_fwd_i8",
           "sla_quantize_i8f8", "sla_sparse_fwd_i8f8",
           "sla_bwd_workspace_bytes", "sla_sparse_bwd", "sla_linear_bwd", "sla_attn_bwd", "sla_attn_bwd_saved",
           "sla_alpha_grad",
           "sla_status_string")


class SlaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({text})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("bq", ctypes.c_int32), ("bk", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Select(ctypes.Structure):
    _fields_ = [("k_frac", ctypes.c_float), ("p", ctypes.c_float),
                ("Wq", ctypes.c_void_p), ("Wk", ctypes.c_void_p)]


class I8Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("q8", "k8", "vt8", "sq", "sk", "sv", "rv", "vpart", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsla.so once (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found; build it with "
                               "`python -m block_sparse_linear_sla_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, vp = ctypes.POINTER(Problem), ctypes.POINTER(Select), ctypes.c_void_p
        L.sla_workspace_bytes.argtypes = [P, S]
        L.sla_workspace_bytes.restype = ctypes.c_size_t
        L.sla_mask_capacity.argtypes = [P]
        L.sla_mask_capacity.restype = ctypes.c_int64
        L.sla_mask.argtypes = [P, S, vp, vp, vp, vp, ctypes.c_int64, vp, vp, ctypes.c_size_t, vp]
        L.sla_mask_prepared.argtypes = [P, S, vp, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_size_t, vp]
        L.sla_soft_topk.argtypes = [P, S, ctypes.c_float, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_mask_noalloc_bytes.argtypes = [P, S]
        L.sla_mask_noalloc_bytes.restype = ctypes.c_size_t
        L.sla_mask_noalloc.argtypes = [P, S, vp, vp, vp, vp, ctypes.c_int64, vp]
        L.sla_sparse_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.sla_linear_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_attn_fwd.argtypes = [P, S, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp,
                                   ctypes.c_size_t, vp]
        L.sla_kv_prepare.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_fused_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_saved_terms_count.argtypes = [P]
        L.sla_saved_terms_count.restype = ctypes.c_int64
        L.sla_fused_fwd_save.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp, vp]
        L.sla_dense_fwd.argtypes = [P, vp, vp, vp, vp, vp]
        L.sla_i8_layout_of.argtypes = [P, ctypes.POINTER(I8Layout)]
        L.sla_quantize_i8.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_sparse_fwd_i8.argtypes = [P, vp, ctypes.c_size_t, vp, vp, vp, vp]
        L.sla_quantize_i8f8.argtypes = [P, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_sparse_fwd_i8f8.argtypes = [P, vp, ctypes.c_size_t, vp, vp, vp, vp]
        L.sla_bwd_workspace_bytes.argtypes = [P]
        L.sla_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.sla_sparse_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_linear_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int, vp, ctypes.c_size_t,
                                     vp]
        L.sla_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_attn_bwd_saved.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        L.sla_alpha_grad.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.sla_status_string.argtypes = [ctypes.c_int]
        L.sla_status_string.restype = ctypes.c_char_p
        for fn in ("sla_mask", "sla_mask_prepared", "sla_mask_noalloc", "sla_soft_topk", "sla_sparse_fwd", "sla_linear_fwd", "sla_attn_fwd",
                   "sla_kv_prepare", "sla_fused_fwd", "sla_fused_fwd_save", "sla_dense_fwd", "sla_i8_layout_of",
                   "sla_quantize_i8", "sla_sparse_fwd_i8", "sla_quantize_i8f8", "sla_sparse_fwd_i8f8",
                   "sla_sparse_bwd", "sla_linear_bwd",
                   "sla_attn_bwd", "sla_attn_bwd_saved", "sla_alpha_grad"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise SlaError(fn, status, lib().sla_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SLA_BF16
    if t.dtype == torch.float32:
        return SLA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def problem(q: torch.Tensor, bq: int, bk: int) -> Problem:
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d]")
    B, H, N, d = q.shape
    return Problem(B, H, N, d, bq, bk, _dtype_code(q))


def select(k_frac: float, p: float, wq: Optional[torch.Tensor] = None,
           wk: Optional[torch.Tensor] = None) -> Select:
    return Select(float(k_frac), float(p), _ptr(wq), _ptr(wk))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(*ts: torch.Tensor, like: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous CUDA tensors")
        if t.shape != like.shape or t.dtype != like.dtype:
            raise ValueError("Q, K, V (and outputs) must share shape and dtype")


def sla_workspace_bytes(prob: Problem, sel: Optional[Select] = None) -> int:
    return int(lib().sla_workspace_bytes(ctypes.byref(prob), ctypes.byref(sel) if sel else None))


def sla_mask_capacity(prob: Problem) -> int:
    return int(lib().sla_mask_capacity(ctypes.byref(prob)))


def workspace(prob: Problem, sel: Optional[Select] = None, device=None) -> torch.Tensor:
    n = sla_workspace_bytes(prob, sel)
    if n == 0:
        raise ValueError("invalid problem")
    return torch.empty(n, dtype=torch.uint8, device=device)


def sla_mask(q, k, bq: int, bk: int, k_frac: float, p: float, wq=None, wk=None,
             return_logits: bool = False, ws: Optional[torch.Tensor] = None,
             row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None):
    """Block mask as CSR: (row_ptr int32 [R+1], col_idx int32 [capacity]) and,
    if asked, the pooled logits (float64 [B, H, Nq, Nk]).  Only the first
    row_ptr[-1] entries of col_idx are meaningful."""
    _need(q, k, like=q)
    prob, sel = problem(q, bq, bk), select(k_frac, p, wq, wk)
    cap = sla_mask_capacity(prob)
    B, H = q.shape[:2]
    Nq, Nk = -(-q.shape[2] // bq), -(-q.shape[2] // bk)
    dev = q.device
    rp = row_ptr if row_ptr is not None else torch.empty(B * H * Nq + 1, dtype=torch.int32, device=dev)
    ci = col_idx if col_idx is not None else torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    logits = torch.empty((B, H, Nq, Nk), dtype=torch.float64, device=dev) if return_logits else None
    w = ws if ws is not None else workspace(prob, sel, dev)
    _check("sla_mask", lib().sla_mask(ctypes.byref(prob), ctypes.byref(sel), _ptr(q), _ptr(k),
                                      _ptr(rp), _ptr(ci), ci.numel(), _ptr(logits), _ptr(w),
                                      w.numel(), _stream()))
    return (rp, ci, logits) if return_logits else (rp, ci)


def sla_mask_noalloc_bytes(prob: Problem, sel: Optional[Select] = None) -> int:
    return int(lib().sla_mask_noalloc_bytes(ctypes.byref(prob), ctypes.byref(sel) if sel else None))


def sla_mask_noalloc(q, k, bq: int, bk: int, k_frac: float, p: float, wq=None, wk=None,
                     row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None):
    """sla_mask with the library's static device scratch instead of a
    workspace (the call itself allocates nothing; the outputs are allocated
    here unless passed in).  Returns (row_ptr, col_idx) as sla_mask."""
    _need(q, k, like=q)
    prob, sel = problem(q, bq, bk), select(k_frac, p, wq, wk)
    cap = sla_mask_capacity(prob)
    B, H = q.shape[:2]
    Nq = -(-q.shape[2] // bq)
    dev = q.device
    rp = row_ptr if row_ptr is not None else torch.empty(B * H * Nq + 1, dtype=torch.int32, device=dev)
    ci = col_idx if col_idx is not None else torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check("sla_mask_noalloc", lib().sla_mask_noalloc(ctypes.byref(prob), ctypes.byref(sel), _ptr(q), _ptr(k),
                                                      _ptr(rp), _ptr(ci), ci.numel(), _stream()))
    return rp, ci


def sla_mask_prepared(q, k, alpha, bq: int, bk: int, k_frac: float, p: float, wq=None, wk=None,
                      ws: Optional[torch.Tensor] = None, row_ptr: Optional[torch.Tensor] = None,
                      col_idx: Optional[torch.Tensor] = None):
    """sla_mask for a workspace on which sla_kv_prepare(k, v, ..., alpha) has
    just run (it pooled K for the heads it processed): the same CSR."""
    _need(q, k, like=q)
    if not alpha.is_cuda or alpha.dtype != torch.float32 or alpha.numel() != q.shape[1]:
        raise ValueError("alpha must be a CUDA float32 tensor of H entries")
    if ws is None:
        raise ValueError("sla_mask_prepared needs the workspace sla_kv_prepare filled")
    prob, sel = problem(q, bq, bk), select(k_frac, p, wq, wk)
    cap = sla_mask_capacity(prob)
    B, H = q.shape[:2]
    Nq = -(-q.shape[2] // bq)
    dev = q.device
    rp = row_ptr if row_ptr is not None else torch.empty(B * H * Nq + 1, dtype=torch.int32, device=dev)
    ci = col_idx if col_idx is not None else torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check("sla_mask_prepared", lib().sla_mask_prepared(ctypes.byref(prob), ctypes.byref(sel), _ptr(q), _ptr(k),
                                                        _ptr(alpha), _ptr(rp), _ptr(ci), ci.numel(), _ptr(ws),
                                                        ws.numel(), _stream()))
    return rp, ci


def sla_soft_topk(q, k, bq: int, bk: int, k_frac: float, T: float, wq=None, wk=None,
                  out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """SoftTop-k weights, float32 [B, H, Nq, Nk] (rows sum to ceil(k_frac * Nk))."""
    _need(q, k, like=q)
    prob, sel = problem(q, bq, bk), select(k_frac, 0.0, wq, wk)
    B, H = q.shape[:2]
    Nq, Nk = -(-q.shape[2] // bq), -(-q.shape[2] // bk)
    m = out if out is not None else torch.empty((B, H, Nq, Nk), dtype=torch.float32, device=q.device)
    w = ws if ws is not None else workspace(prob, sel, q.device)
    _check("sla_soft_topk", lib().sla_soft_topk(ctypes.byref(prob), ctypes.byref(sel), float(T), _ptr(q),
                                                _ptr(k), _ptr(m), _ptr(w), w.numel(), _stream()))
    return m


def sla_sparse_fwd(q, k, v, bq: int, bk: int, row_ptr, col_idx, out=None):
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    o = out if out is not None else torch.empty_like(q)
    _check("sla_sparse_fwd", lib().sla_sparse_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                                  _ptr(row_ptr), _ptr(col_idx), _ptr(o), _stream()))
    return o


def sla_linear_fwd(q, k, v, bq: int, bk: int, row_ptr, col_idx, out=None, ws=None):
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    o = out if out is not None else torch.empty_like(q)
    w = ws if ws is not None else workspace(prob, None, q.device)
    _check("sla_linear_fwd", lib().sla_linear_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                                  _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(w),
                                                  w.numel(), _stream()))
    return o


def sla_attn_fwd(q, k, v, alpha, bq: int, bk: int, k_frac: float, p: float, wq=None, wk=None,
                 out=None, ws=None, row_ptr=None, col_idx=None) -> Tuple[torch.Tensor, ...]:
    """Whole forward.  Returns (O, row_ptr, col_idx)."""
    _need(q, k, v, like=q)
    if not alpha.is_cuda or alpha.dtype != torch.float32 or alpha.numel() != q.shape[1]:
        raise ValueError("alpha must be a CUDA float32 tensor of H entries")
    prob, sel = problem(q, bq, bk), select(k_frac, p, wq, wk)
    cap = sla_mask_capacity(prob)
    B, H = q.shape[:2]
    Nq = -(-q.shape[2] // bq)
    dev = q.device
    o = out if out is not None else torch.empty_like(q)
    rp = row_ptr if row_ptr is not None else torch.empty(B * H * Nq + 1, dtype=torch.int32, device=dev)
    ci = col_idx if col_idx is not None else torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    w = ws if ws is not None else workspace(prob, sel, dev)
    _check("sla_attn_fwd", lib().sla_attn_fwd(ctypes.byref(prob), ctypes.byref(sel), _ptr(q), _ptr(k),
                                              _ptr(v), _ptr(alpha), _ptr(o), _ptr(rp), _ptr(ci),
                                              ci.numel(), _ptr(w), w.numel(), _stream()))
    return o, rp, ci


def sla_kv_prepare(k, v, bq: int, bk: int, ws: torch.Tensor, alpha=None):
    """One pass over K and V leaving in ws what sla_fused_fwd reads."""
    _need(k, v, like=k)
    prob = problem(k, bq, bk)
    _check("sla_kv_prepare", lib().sla_kv_prepare(ctypes.byref(prob), _ptr(k), _ptr(v), _ptr(alpha),
                                                  _ptr(ws), ws.numel(), _stream()))


def sla_fused_fwd(q, k, v, alpha, bq: int, bk: int, row_ptr, col_idx, ws: torch.Tensor, out=None):
    """alpha-mixed sparse + linear output over a given mask, reading the totals
    that sla_kv_prepare left in ws."""
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    o = out if out is not None else torch.empty_like(q)
    _check("sla_fused_fwd", lib().sla_fused_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(alpha), _ptr(row_ptr), _ptr(col_idx), _ptr(o),
                                                _ptr(ws), ws.numel(), _stream()))
    return o


def sla_saved_terms_count(prob: Problem) -> int:
    return int(lib().sla_saved_terms_count(ctypes.byref(prob)))


def sla_fused_fwd_save(q, k, v, alpha, bq: int, bk: int, row_ptr, col_idx, ws: torch.Tensor, out=None,
                       saved=None):
    """sla_fused_fwd that also keeps, for the backward of a training step,
    each query's normalisers and the two branch outputs (float32).  Returns
    (O, saved) with saved = dict(lse2, invden, o_s, o_l)."""
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    o = out if out is not None else torch.empty_like(q)
    if saved is None:
        n = sla_saved_terms_count(prob)
        saved = dict(lse2=torch.empty(max(n, 1), dtype=torch.float32, device=q.device),
                     invden=torch.empty(max(n, 1), dtype=torch.float32, device=q.device),
                     o_s=torch.empty(q.shape, dtype=torch.float32, device=q.device),
                     o_l=torch.empty(q.shape, dtype=torch.float32, device=q.device))
    _check("sla_fused_fwd_save", lib().sla_fused_fwd_save(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(row_ptr), _ptr(col_idx), _ptr(o),
        _ptr(ws), ws.numel(), _ptr(saved["lse2"]), _ptr(saved["invden"]), _ptr(saved["o_s"]),
        _ptr(saved["o_l"]), _stream()))
    return o, saved


def sla_dense_fwd(q, k, v, bq: int = 128, bk: int = 64, out=None):
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    o = out if out is not None else torch.empty_like(q)
    _check("sla_dense_fwd", lib().sla_dense_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                                _stream()))
    return o


# ------------------------------------------------------- 8-bit sparse branch
def sla_i8_layout_of(prob: Problem) -> I8Layout:
    lay = I8Layout()
    _check("sla_i8_layout_of", lib().sla_i8_layout_of(ctypes.byref(prob), ctypes.byref(lay)))
    return lay


def sla_quantize_i8(q, k, v, bq: int, bk: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """8-bit codes and scales of Q, K, V in one uint8 buffer (layout from
    sla_i8_layout_of; i8_views splits it)."""
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    n = sla_i8_layout_of(prob).total
    buf = out if out is not None else torch.empty(n, dtype=torch.uint8, device=q.device)
    _check("sla_quantize_i8", lib().sla_quantize_i8(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(buf),
                                                    buf.numel(), _stream()))
    return buf


def sla_sparse_fwd_i8(qbuf: torch.Tensor, like: torch.Tensor, bq: int, bk: int, row_ptr, col_idx,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The 8-bit sparse branch over the codes in qbuf; `like` gives the shape,
    dtype and device of Q (its data is not read)."""
    prob = problem(like, bq, bk)
    o = out if out is not None else torch.empty_like(like)
    _check("sla_sparse_fwd_i8", lib().sla_sparse_fwd_i8(ctypes.byref(prob), _ptr(qbuf), qbuf.numel(),
                                                        _ptr(row_ptr), _ptr(col_idx), _ptr(o), _stream()))
    return o


def sla_quantize_i8f8(q, k, v, bq: int, bk: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 Q, K and E4M3 V codes and their scales in one uint8 buffer (the
    layout of sla_i8_layout_of; i8_views splits it, vt8 as E4M3 bytes)."""
    _need(q, k, v, like=q)
    prob = problem(q, bq, bk)
    n = sla_i8_layout_of(prob).total
    buf = out if out is not None else torch.empty(n, dtype=torch.uint8, device=q.device)
    _check("sla_quantize_i8f8", lib().sla_quantize_i8f8(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(buf),
                                                      buf.numel(), _stream()))
    return buf


def sla_sparse_fwd_i8f8(qbuf: torch.Tensor, like: torch.Tensor, bq: int, bk: int, row_ptr, col_idx,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The single-pass 8-bit sparse branch (int8 scores, E4M3 P and V) over
    the codes in qbuf; `like` gives the shape, dtype and device of Q (its data
    is not read)."""
    prob = problem(like, bq, bk)
    o = out if out is not None else torch.empty_like(like)
    _check("sla_sparse_fwd_i8f8", lib().sla_sparse_fwd_i8f8(ctypes.byref(prob), _ptr(qbuf), qbuf.numel(),
                                                          _ptr(row_ptr), _ptr(col_idx), _ptr(o), _stream()))
    return o


def i8_views(qbuf: torch.Tensor, shape, bq: int, bk: int, dtype=torch.bfloat16) -> dict:
    """Views of the regions of a quantised buffer: q8 [BH, Nq*bq, d], k8
    [BH, Nk*bk, d], vt8 [BH, Nk*bk/64, d, 64] (int8), sq [BH, Nq], sk [BH, Nk],
    sv and rv [BH, d] (float32)."""
    B, H, N, d = shape
    prob = Problem(B, H, N, d, bq, bk, SLA_BF16 if dtype == torch.bfloat16 else SLA_F32)
    lay = sla_i8_layout_of(prob)
    BH, Nq, Nk = B * H, -(-N // bq), -(-N // bk)

    def region(off, count, dt):
        nbytes = count * torch.empty((), dtype=dt).element_size()
        return qbuf[off:off + nbytes].view(dt)

    return {
        "q8": region(lay.q8, BH * Nq * bq * d, torch.int8).view(BH, Nq * bq, d),
        "k8": region(lay.k8, BH * Nk * bk * d, torch.int8).view(BH, Nk * bk, d),
        "vt8": region(lay.vt8, BH * Nk * bk * d, torch.int8).view(BH, Nk * bk // 64, d, 64),
        "sq": region(lay.sq, BH * Nq, torch.float32).view(BH, Nq),
        "sk": region(lay.sk, BH * Nk, torch.float32).view(BH, Nk),
        "sv": region(lay.sv, BH * d, torch.float32).view(BH, d),
        "rv": region(lay.rv, BH * d, torch.float32).view(BH, d),
    }


# ------------------------------------------------------------------ backward
def sla_bwd_workspace_bytes(prob: Problem) -> int:
    return int(lib().sla_bwd_workspace_bytes(ctypes.byref(prob)))


def bwd_workspace(prob: Problem, device=None) -> torch.Tensor:
    n = sla_bwd_workspace_bytes(prob)
    if n == 0:
        raise ValueError("invalid problem")
    return torch.empty(n, dtype=torch.uint8, device=device)


def sla_sparse_bwd(q, k, v, do_s, bq: int, bk: int, row_ptr, col_idx, ws=None, out=None):
    """Gradient of sum(O_s * dO_s) with the mask fixed: returns (dQ, dK, dV)."""
    _need(q, k, v, do_s, like=q)
    prob = problem(q, bq, bk)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    w = ws if ws is not None else bwd_workspace(prob, q.device)
    _check("sla_sparse_bwd", lib().sla_sparse_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do_s), _ptr(row_ptr), _ptr(col_idx), _ptr(dq), _ptr(dk),
                                                  _ptr(dv), _ptr(w), w.numel(), _stream()))
    return dq, dk, dv


def sla_linear_bwd(q, k, v, do_l, bq: int, bk: int, row_ptr, col_idx, ws=None, out=None,
                   accumulate: bool = False):
    """Gradient of sum(O_l * dO_l), the linear branch over the unselected
    blocks, with the mask fixed: returns (dQ, dK, dV).  With accumulate the
    results are added into `out` (for example the sparse branch's gradient)."""
    _need(q, k, v, do_l, like=q)
    prob = problem(q, bq, bk)
    if accumulate and out is None:
        raise ValueError("accumulate needs the out buffers")
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    w = ws if ws is not None else bwd_workspace(prob, q.device)
    _check("sla_linear_bwd", lib().sla_linear_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do_l),
                                                  _ptr(row_ptr), _ptr(col_idx), _ptr(dq), _ptr(dk), _ptr(dv),
                                                  1 if accumulate else 0, _ptr(w), w.numel(), _stream()))
    return dq, dk, dv


def sla_attn_bwd(q, k, v, do, alpha, bq: int, bk: int, row_ptr, col_idx, ws=None, out=None, dalpha=None):
    """Gradient of sum(O * dO) for O = alpha_h O_s + (1 - alpha_h) O_l with
    the mask fixed: returns (dQ, dK, dV); with dalpha (float32 [H] CUDA
    tensor) the alpha gradient is written there as well."""
    _need(q, k, v, do, like=q)
    if alpha.dtype != torch.float32 or not alpha.is_cuda or alpha.numel() != q.shape[1]:
        raise ValueError("alpha must be a float32 CUDA tensor of H values")
    prob = problem(q, bq, bk)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    w = ws if ws is not None else bwd_workspace(prob, q.device)
    _check("sla_attn_bwd", lib().sla_attn_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do),
                                              _ptr(alpha.contiguous()), _ptr(row_ptr), _ptr(col_idx), _ptr(dq),
                                              _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(w), w.numel(), _stream()))
    return dq, dk, dv


def sla_attn_bwd_saved(q, k, v, do, alpha, bq: int, bk: int, row_ptr, col_idx, saved, ws=None, out=None,
                       dalpha=None):
    """sla_attn_bwd reading the terms sla_fused_fwd_save kept (saved: its
    dict) instead of recomputing them: returns (dQ, dK, dV, dalpha) with
    dalpha the alpha gradient (float32 [H])."""
    _need(q, k, v, do, like=q)
    for t in (saved["o_s"], saved["o_l"]):
        if t.dtype != torch.float32 or t.shape != q.shape or not t.is_cuda or not t.is_contiguous():
            raise ValueError("the saved branch outputs must be contiguous float32 CUDA tensors shaped like Q")
    if alpha.dtype != torch.float32 or not alpha.is_cuda or alpha.numel() != q.shape[1]:
        raise ValueError("alpha must be a float32 CUDA tensor of H values")
    prob = problem(q, bq, bk)
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    da = dalpha if dalpha is not None else torch.empty(q.shape[1], dtype=torch.float32, device=q.device)
    w = ws if ws is not None else bwd_workspace(prob, q.device)
    _check("sla_attn_bwd_saved", lib().sla_attn_bwd_saved(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(alpha.contiguous()), _ptr(row_ptr),
        _ptr(col_idx), _ptr(saved["lse2"]), _ptr(saved["invden"]), _ptr(saved["o_s"]), _ptr(saved["o_l"]),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(w), w.numel(), _stream()))
    return dq, dk, dv, da


def sla_alpha_grad(do, o_s, o_l, bq: int = 128, bk: int = 64, ws=None) -> torch.Tensor:
    """d/d alpha of sum(O * dO), O = alpha_h O_s + (1 - alpha_h) O_l: float32 [H]."""
    _need(do, o_s, o_l, like=do)
    prob = problem(do, bq, bk)
    da = torch.empty(do.shape[1], dtype=torch.float32, device=do.device)
    w = ws if ws is not None else bwd_workspace(prob, do.device)
    _check("sla_alpha_grad", lib().sla_alpha_grad(ctypes.byref(prob), _ptr(do), _ptr(o_s), _ptr(o_l), _ptr(da),
                                                  _ptr(w), w.numel(), _stream()))
    return da
