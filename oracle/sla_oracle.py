"""Plain float64 CPU oracle for the sparse + linear attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it.  It shares no code, constant or helper with the HIP
library: it computes every step from its definition, slowly and directly, so
that a reader can check it against the sources by eye.

Sources (cited by short key):

* [SA2 §n]  - the web write-up of SpargeAttention2 (arXiv:2602.13515) titled
  "清華發明AI「注意力瘦身術」：視頻生成速度提升16倍的神奇技術", section n
  (§一 the hybrid Top-k / Top-p mask, §四 the pool -> select -> block pipeline,
  §六 why the two selection rules fail in opposite regimes).
* [SLA2 §n] - the web write-up of SLA2 (arXiv:2602.12675), section n
  (§一 sparse branch for important regions, linear branch for the rest;
  §二 the learnable mixing ratio and the two-matrix learnable router).
* [DEF] - the textbook dense attention softmax(Q K^T / sqrt(d)) V, which is the
  only formula the pages print.
* [FM]  - the feature map phi(x) = elu(x) + 1 of Katharopoulos et al. 2020,
  "Transformers are RNNs", used for the linear branch.

Readings taken where the pages are silent:

* pooled scores use the attention scale 1/sqrt(d); P is a row softmax;
* k = ceil(k_frac * Nk - 1e-9) from float32 k_frac widened to float64;
* Top-p keeps the item whose cumulative mass first reaches p (inclusive);
  p <= 0 keeps nothing; if p is never reached every block is kept;
* ties are broken toward the lower block index, in one order shared by both
  rules, so the union is the longer prefix of that order;
* the last block of a sequence may be partial: pooling divides by the true
  count and keys past N do not exist for either branch;
* the router is a row vector times a [d, d] matrix, shared by all heads;
* the linear branch is normalised over the unselected keys only, with no
  1/sqrt(d); it is 0 when every block is selected, and the sparse branch is 0
  when none is;
* O = alpha_h * O_sparse + (1 - alpha_h) * O_linear per head.

Every function works on float64 numpy arrays; inputs given in bf16/fp32 are
widened exactly, so input rounding is never mistaken for kernel error.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


def as_f64(x) -> np.ndarray:
    """Widen a torch tensor (any float dtype) or array to float64 exactly."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- partition
def n_blocks(N: int, b: int) -> int:
    """Number of blocks of size b covering N tokens; the last may be partial
    [SA2 §四: the computation is cut into small blocks]."""
    return -(-N // b)


def block_range(i: int, b: int, N: int) -> Tuple[int, int]:
    """Token range [start, end) of block i."""
    return i * b, min((i + 1) * b, N)


# ---------------------------------------------------------------- pooling
def pool(X: np.ndarray, b: int) -> np.ndarray:
    """Block mean pooling of one head's [N, d] rows -> [ceil(N/b), d]
    [SA2 §四: neighbouring tokens are merged into a quick overview].
    The mean divides the block's sum by its true token count."""
    N, d = X.shape
    nb = n_blocks(N, b)
    out = np.empty((nb, d), dtype=np.float64)
    for i in range(nb):
        s, e = block_range(i, b, N)
        out[i] = X[s:e].sum(axis=0) / float(e - s)
    return out


def route(xbar: np.ndarray, W: Optional[np.ndarray]) -> np.ndarray:
    """Learned router projection of pooled vectors, row vector times matrix
    [SLA2 §二: two learnable projection matrices map query and key features
    into a space suited to routing].  Identity when W is None."""
    if W is None:
        return xbar
    return xbar @ W


def block_scores(qhat: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """Pooled block logits S_ij = qhat_i . khat_j / sqrt(d) [DEF]."""
    d = qhat.shape[1]
    return (qhat @ khat.T) / math.sqrt(d)


def row_softmax(S: np.ndarray) -> np.ndarray:
    """P_ij = exp(S_ij - max_j S_ij) / sum_j exp(S_ij - max_j S_ij)."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- selection
def k_from_frac(k_frac: float, Nk: int) -> int:
    """Top-k count: at least the fraction k_frac of the key blocks.
    k_frac is taken as the float32 the C interface receives."""
    kf = float(np.float32(k_frac))
    k = math.ceil(kf * Nk - 1e-9)
    return max(0, min(Nk, k))


def block_order(P_row: np.ndarray) -> np.ndarray:
    """Block indices by probability, largest first, ties to the lower index."""
    Nk = len(P_row)
    return np.lexsort((np.arange(Nk), -P_row))


def topk_count(k: int, Nk: int) -> int:
    """Top-k keeps a fixed number of blocks whatever the distribution
    [SA2 §一: a fixed number, e.g. always 3]."""
    return max(0, min(Nk, k))


def topp_count(P_sorted: np.ndarray, p: float) -> int:
    """Top-p keeps blocks in order until their cumulative importance reaches
    the threshold p [SA2 §一: keep adding until the sum reaches e.g. 60%].
    Returns the smallest n with sum of the first n >= p (inclusive reading);
    0 when p <= 0; every block when p is never reached."""
    p64 = float(np.float32(p))
    if p64 <= 0.0:
        return 0
    c = np.cumsum(P_sorted)
    hit = np.nonzero(c >= p64)[0]
    return int(hit[0]) + 1 if len(hit) else len(P_sorted)


def select_row(P_row: np.ndarray, k: int, p: float) -> Tuple[np.ndarray, Dict]:
    """Hybrid selection for one query block: the union of the Top-k set and
    the Top-p set [SA2 §一: run both rules, then merge their results].
    Both sets are prefixes of the same order, so the union is the prefix of
    length max(k, kp).  Returns ascending block indices and diagnostics."""
    order = block_order(P_row)
    Ps = P_row[order]
    kk = topk_count(k, len(P_row))
    kp = topp_count(Ps, p)
    n = max(kk, kp)
    info = dict(order=order, cum=np.cumsum(Ps), k=kk, kp=kp, n=n)
    return np.sort(order[:n]), info


# ---------------------------------------------------------------- mask
def mask(Q, K, bq: int, bk: int, k_frac: float, p: float, Wq=None, Wk=None,
         keep_info: bool = True):
    """Block mask of every (b, h, query block) as CSR.

    Q, K: [B, H, N, d].  Rows are ordered (b, h, i); column indices ascending.
    Returns (row_ptr int64 [R+1], col_idx int64 [nnz], info) where info holds,
    per row, the logits S, the probabilities P, the order, the cumulative sums
    and the counts (used to excuse blocks that sit on the selection cut).
    [SA2 §四: pool -> hybrid select on the pooled map -> block-level mask
    marking each block important or negligible.]
    """
    Q = as_f64(Q)
    K = as_f64(K)
    Wq = None if Wq is None else as_f64(Wq)
    Wk = None if Wk is None else as_f64(Wk)
    B, H, N, d = Q.shape
    Nq, Nk = n_blocks(N, bq), n_blocks(N, bk)
    k = k_from_frac(k_frac, Nk)
    counts: List[int] = []
    cols: List[np.ndarray] = []
    S_all = np.empty((B, H, Nq, Nk))
    P_all = np.empty((B, H, Nq, Nk))
    rows_info = []
    for b in range(B):
        for h in range(H):
            qhat = route(pool(Q[b, h], bq), Wq)
            khat = route(pool(K[b, h], bk), Wk)
            S = block_scores(qhat, khat)
            P = row_softmax(S)
            S_all[b, h] = S
            P_all[b, h] = P
            for i in range(Nq):
                sel, info = select_row(P[i], k, p)
                counts.append(len(sel))
                cols.append(sel)
                if keep_info:
                    rows_info.append(info)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int64) if cols else np.zeros(0, np.int64)
    meta = dict(S=S_all, P=P_all, rows=rows_info, k=k, Nq=Nq, Nk=Nk)
    return row_ptr, col_idx, meta


# ---------------------------------------------------------------- SoftTop-k
def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function 1 / (1 + exp(-x)), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def soft_topk_row(S_row: np.ndarray, k: int, T: float) -> Tuple[np.ndarray, float]:
    """SoftTop-k of one row of pooled logits [SLA2 §四: in the router's first
    training stage the hard Top-k is replaced by a SoftTop-k made of a sigmoid
    with a temperature, which lets gradients through].

    Reading (the pages name only the sigmoid and the temperature): the soft
    weight of block j is M_j = sigmoid((S_j - tau) / T), with the one threshold
    tau for which the weights sum to k, so the soft mask keeps k blocks' worth
    of weight and tends to the hard Top-k indicator as T -> 0.  k = 0 gives all
    zeros and k = Nk all ones (tau = +inf / -inf).  tau is found by bisection
    on the decreasing function f(tau) = sum_j sigmoid((S_j - tau) / T) - k,
    run until the bracket stops shrinking.  Returns (M, tau)."""
    S_row = np.asarray(S_row, dtype=np.float64)
    Nk = len(S_row)
    if k <= 0:
        return np.zeros(Nk), math.inf
    if k >= Nk:
        return np.ones(Nk), -math.inf
    lo = float(S_row.min()) - 80.0 * T   # f(lo) > 0: every weight ~ 1
    hi = float(S_row.max()) + 80.0 * T   # f(hi) < 0: every weight ~ 0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if sigmoid((S_row - mid) / T).sum() > k:
            lo = mid
        else:
            hi = mid
    tau = 0.5 * (lo + hi)
    return sigmoid((S_row - tau) / T), tau


def soft_topk(Q, K, bq: int, bk: int, k_frac: float, T: float, Wq=None, Wk=None) -> np.ndarray:
    """SoftTop-k mask of every (b, h, query block): [B, H, Nq, Nk] weights from
    the pooled (and optionally routed) block logits, k = ceil(k_frac * Nk)
    as for the hard mask."""
    Q = as_f64(Q)
    K = as_f64(K)
    Wq = None if Wq is None else as_f64(Wq)
    Wk = None if Wk is None else as_f64(Wk)
    B, H, N, d = Q.shape
    Nq, Nk = n_blocks(N, bq), n_blocks(N, bk)
    k = k_from_frac(k_frac, Nk)
    M = np.empty((B, H, Nq, Nk))
    for b in range(B):
        for h in range(H):
            S = block_scores(route(pool(Q[b, h], bq), Wq), route(pool(K[b, h], bk), Wk))
            for i in range(Nq):
                M[b, h, i], _ = soft_topk_row(S[i], k, T)
    return M


# ---------------------------------------------------------------- branches
def _keys_of(blocks: Iterable[int], bk: int, N: int) -> np.ndarray:
    """Token indices of the given key blocks (partial last block clipped)."""
    idx = [np.arange(*block_range(int(j), bk, N)) for j in blocks]
    return np.concatenate(idx) if idx else np.zeros(0, dtype=np.int64)


def phi(x: np.ndarray) -> np.ndarray:
    """Linear-attention feature map elu(x) + 1 [FM]: x + 1 for x > 0, exp(x)
    otherwise (always positive)."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _rows(B: int, H: int, Nq: int, rows):
    if rows is None:
        return [(b, h, i) for b in range(B) for h in range(H) for i in range(Nq)]
    return list(rows)


def sparse_branch(Q, K, V, bq: int, bk: int, row_ptr, col_idx, rows=None) -> Dict:
    """Exact softmax attention of each query token over the keys of its
    block's selected key blocks only, renormalised over them
    [SLA2 §一: important regions get precise sparse attention; SLA2 §二: the
    sparse branch renormalises over what it keeps].  Two-pass softmax
    (max, then exp / sum).  Zero when no block is selected.
    Returns {(b, h, i): [rows_in_block, d]} for the requested rows."""
    Q, K, V = as_f64(Q), as_f64(K), as_f64(V)
    B, H, N, d = Q.shape
    Nq = n_blocks(N, bq)
    out = {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        s, e = block_range(i, bq, N)
        keys = _keys_of(sel, bk, N)
        if len(keys) == 0:
            out[(b, h, i)] = np.zeros((e - s, d))
            continue
        Sx = Q[b, h, s:e] @ K[b, h, keys].T / math.sqrt(d)
        m = Sx.max(axis=1, keepdims=True)
        E = np.exp(Sx - m)
        out[(b, h, i)] = (E @ V[b, h, keys]) / E.sum(axis=1, keepdims=True)
    return out


def linear_branch(Q, K, V, bq: int, bk: int, row_ptr, col_idx, rows=None) -> Dict:
    """Linear attention of each query token over the keys of the key blocks
    its block did NOT select [SLA2 §一: the less important regions go to the
    cheaper linear attention], by direct summation:
        O_l(t) = sum_u (phi(q_t).phi(k_u)) v_u / sum_u phi(q_t).phi(k_u)
    over the unselected keys u.  Zero when every block is selected."""
    Q, K, V = as_f64(Q), as_f64(K), as_f64(V)
    B, H, N, d = Q.shape
    Nq, Nk = n_blocks(N, bq), n_blocks(N, bk)
    out = {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = set(int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]])
        unsel = [j for j in range(Nk) if j not in sel]
        s, e = block_range(i, bq, N)
        keys = _keys_of(unsel, bk, N)
        if len(keys) == 0:
            out[(b, h, i)] = np.zeros((e - s, d))
            continue
        A = phi(Q[b, h, s:e]) @ phi(K[b, h, keys]).T
        out[(b, h, i)] = (A @ V[b, h, keys]) / A.sum(axis=1, keepdims=True)
    return out


def sparse_branch_lse(Q, K, bq: int, bk: int, row_ptr, col_idx, rows=None) -> Dict:
    """Natural log of each query's sparse-branch softmax normaliser,
        lse(t) = log sum_u exp(q_t . k_u / sqrt(d))
    over the keys u of its block's selected key blocks [SLA2 §一; DEF]: the
    value a backward pass needs to recover the branch's probabilities,
    exp(q_t . k_u / sqrt(d) - lse(t)).  -inf (the log of an empty sum) when
    no block is selected.  Returns {(b, h, i): [rows_in_block]}."""
    Q, K = as_f64(Q), as_f64(K)
    B, H, N, d = Q.shape
    Nq = n_blocks(N, bq)
    out = {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        s, e = block_range(i, bq, N)
        keys = _keys_of(col_idx[row_ptr[r]:row_ptr[r + 1]], bk, N)
        if len(keys) == 0:
            out[(b, h, i)] = np.full(e - s, -np.inf)
            continue
        Sx = Q[b, h, s:e] @ K[b, h, keys].T / math.sqrt(d)
        m = Sx.max(axis=1)
        out[(b, h, i)] = m + np.log(np.exp(Sx - m[:, None]).sum(axis=1))
    return out


def linear_branch_den(Q, K, bq: int, bk: int, row_ptr, col_idx, rows=None) -> Dict:
    """Each query's linear-branch normaliser,
        den(t) = sum_u phi(q_t) . phi(k_u)
    over the keys u of the key blocks its block did not select [SLA2 §一;
    FM]; 0 when every block is selected.  Returns {(b, h, i): [rows_in_block]}."""
    Q, K = as_f64(Q), as_f64(K)
    B, H, N, d = Q.shape
    Nq, Nk = n_blocks(N, bq), n_blocks(N, bk)
    out = {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = set(int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]])
        s, e = block_range(i, bq, N)
        keys = _keys_of([j for j in range(Nk) if j not in sel], bk, N)
        out[(b, h, i)] = phi(Q[b, h, s:e]) @ phi(K[b, h, keys]).sum(axis=0) if len(keys) else np.zeros(e - s)
    return out


def combine(Os: np.ndarray, Ol: np.ndarray, alpha_h: float) -> np.ndarray:
    """O = alpha * O_sparse + (1 - alpha) * O_linear [SLA2 §二: the final
    result is the ratio times the sparse result plus one minus the ratio times
    the linear result]."""
    a = float(alpha_h)
    return a * Os + (1.0 - a) * Ol


def attn(Q, K, V, alpha, bq: int, bk: int, row_ptr, col_idx, rows=None) -> Dict:
    """Full forward output for the requested rows given a mask (CSR).
    Branches whose weight is exactly zero are not evaluated."""
    alpha = as_f64(alpha)
    Qa = as_f64(Q)
    B, H, N, d = Qa.shape
    Nq = n_blocks(N, bq)
    rows = _rows(B, H, Nq, rows)
    need_s = [r for r in rows if alpha[r[1]] != 0.0]
    need_l = [r for r in rows if alpha[r[1]] != 1.0]
    Os = sparse_branch(Qa, K, V, bq, bk, row_ptr, col_idx, need_s) if need_s else {}
    Ol = linear_branch(Qa, K, V, bq, bk, row_ptr, col_idx, need_l) if need_l else {}
    out = {}
    for (b, h, i) in rows:
        s, e = block_range(i, bq, N)
        zero = np.zeros((e - s, d))
        out[(b, h, i)] = combine(Os.get((b, h, i), zero), Ol.get((b, h, i), zero), alpha[h])
    return out


def dense(Q, K, V, rows: Optional[Sequence[Tuple[int, int, int]]] = None, bq: int = 128) -> Dict:
    """Dense attention softmax(Q K^T / sqrt(d)) V [DEF], per query block of
    size bq (the blocking only selects which outputs to compute)."""
    Q, K, V = as_f64(Q), as_f64(K), as_f64(V)
    B, H, N, d = Q.shape
    Nq = n_blocks(N, bq)
    out = {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        s, e = block_range(i, bq, N)
        Sx = Q[b, h, s:e] @ K[b, h].T / math.sqrt(d)
        m = Sx.max(axis=1, keepdims=True)
        E = np.exp(Sx - m)
        out[(b, h, i)] = (E @ V[b, h]) / E.sum(axis=1, keepdims=True)
    return out


def assemble(blocks: Dict, B: int, H: int, N: int, d: int, bq: int) -> np.ndarray:
    """Place per-row outputs into a [B, H, N, d] array (NaN where not computed)."""
    out = np.full((B, H, N, d), np.nan)
    for (b, h, i), v in blocks.items():
        s, e = block_range(i, bq, N)
        out[b, h, s:e] = v
    return out


# ------------------------------------------------------- 8-bit sparse branch
# [SLA2 §三]: the sparse branch runs with the query, key, attention-probability
# and value matrices held as 8-bit integers; values are scaled into the 8-bit
# range, the products are formed there, and the results are scaled back.  The
# pages fix neither the scale granularity nor the rounding; the readings taken
# here are:
#
# * symmetric codes in [-127, 127], code = round-half-even(x * (127 / amax)),
#   the reciprocal and the product each rounded to float32, scale = amax / 127
#   (float32); amax = 0 gives scale 0 and zero codes;
# * Q per query block and K per key block (one scale per block of each head),
#   V per channel over the whole sequence of a head (one scale per d index);
# * scores I = q8 . k8 exactly (integers), S = fl32(I * c) with
#   c = fl32(fl32(sq * sk) * fl32(1 / sqrt(d)));  m = the row's maximum S over
#   its selected keys;
# * P codes in [0, 127]: round-half-even(127 exp(S - m)), the value taken in
#   float32 as exp2(fma(I, a, -b)) with a = fl32(c log2 e) and
#   b = fl32(fl32(m log2 e) - log2 127) (a code is an integer decided by
#   floating point, so it is decided in the precision the kernel uses);
# * O = sv * (sum_j code_j v8_j) / (sum_j code_j): numerator and denominator
#   are exact integers; a row with no selected block gives 0.
_F32 = np.float32
_LOG2E_F32 = _F32(math.log2(math.e))
_LOG2_127_F32 = _F32(math.log2(127.0))


def _as_f32_exact(x) -> np.ndarray:
    """Stored bf16 / fp32 values as float32 (exact: both fit)."""
    a = as_f64(x)
    f = a.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), a), "input not representable in float32"
    return f


def quant_codes(x32: np.ndarray, amax: np.float32) -> Tuple[np.ndarray, np.float32]:
    """Symmetric 8-bit codes of float32 values x32 sharing one absolute maximum
    amax, and their scale: code = rint(x * fl32(127 / amax)) in [-127, 127],
    scale = fl32(amax / 127) (zero codes and scale when amax is 0)."""
    amax = _F32(amax)
    if amax == 0:
        return np.zeros(x32.shape, dtype=np.int8), _F32(0.0)
    r = _F32(_F32(127.0) / amax)
    c = np.rint((x32 * r).astype(np.float32))
    return np.clip(c, -127, 127).astype(np.int8), _F32(amax / _F32(127.0))


def quantize_blocks(X, b: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-block codes of X [B, H, N, d]: one scale per (b, h, block of b rows)
    over the block's valid rows and every d.  Returns (codes int8 [B, H, N, d],
    scales float32 [B, H, ceil(N / b)])."""
    X = _as_f32_exact(X)
    B, H, N, d = X.shape
    nb = n_blocks(N, b)
    codes = np.zeros((B, H, N, d), dtype=np.int8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for bb in range(B):
        for h in range(H):
            for i in range(nb):
                s, e = block_range(i, b, N)
                blk = X[bb, h, s:e]
                codes[bb, h, s:e], scales[bb, h, i] = quant_codes(blk, np.abs(blk).max())
    return codes, scales


def quantize_channels(V) -> Tuple[np.ndarray, np.ndarray]:
    """Per-channel codes of V [B, H, N, d]: one scale per (b, h, d index) over
    all N rows.  Returns (codes int8 [B, H, N, d], scales float32 [B, H, d])."""
    V = _as_f32_exact(V)
    B, H, N, d = V.shape
    codes = np.zeros((B, H, N, d), dtype=np.int8)
    scales = np.zeros((B, H, d), dtype=np.float32)
    for bb in range(B):
        for h in range(H):
            for c in range(d):
                col = V[bb, h, :, c]
                codes[bb, h, :, c], scales[bb, h, c] = quant_codes(col, np.abs(col).max())
    return codes, scales


def quantize_i8(Q, K, V, bq: int, bk: int) -> Dict:
    """The 8-bit inputs of the sparse branch [SLA2 §三]: Q per query block,
    K per key block, V per channel."""
    q8, sq = quantize_blocks(Q, bq)
    k8, sk = quantize_blocks(K, bk)
    v8, sv = quantize_channels(V)
    return {"q8": q8, "sq": sq, "k8": k8, "sk": sk, "v8": v8, "sv": sv}


def p_codes(I: np.ndarray, c: np.ndarray, m: np.float32) -> np.ndarray:
    """8-bit codes round-half-even(127 exp(S - m)) of integer scores I with
    per-key score scales c (S = fl32(I c)), evaluated in float32 as
    exp2(fma(I, a, -b)), a = fl32(c log2 e), b = fl32(fl32(m log2 e) - log2 127).
    The fma is exact in float64 before its one rounding to float32; exp2 is
    taken in float64 and rounded to float32."""
    a = (c.astype(np.float32) * _LOG2E_F32).astype(np.float32)
    b = _F32(_F32(_F32(m) * _LOG2E_F32) - _LOG2_127_F32)
    t = (I.astype(np.float64) * a.astype(np.float64) - np.float64(b)).astype(np.float32)
    p = np.exp2(t.astype(np.float64)).astype(np.float32)
    codes = np.rint(p)
    assert codes.max(initial=0) <= 127 and codes.min(initial=0) >= 0
    return codes.astype(np.int64)


def sparse_branch_i8(qz: Dict, bq: int, bk: int, row_ptr, col_idx, rows=None, with_sums: bool = False):
    """The sparse branch on 8-bit codes [SLA2 §三]: for each query of a row
    block, integer scores against the keys of its selected blocks, P codes
    relative to the exact row maximum, and O = sv * sum(code v8) / sum(code)
    from exact integer sums.  Returns {(b, h, i): [rows_in_block, d]}, and with
    with_sums also {(b, h, i): sum of the P codes per query} (0 for an empty
    row)."""
    q8, k8, v8 = (qz[k].astype(np.int64) for k in ("q8", "k8", "v8"))
    sq, sk, sv = qz["sq"], qz["sk"], qz["sv"]
    B, H, N, d = q8.shape
    Nq = n_blocks(N, bq)
    lam = _F32(1.0 / math.sqrt(d))
    out, sums = {}, {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = [int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]]]
        s, e = block_range(i, bq, N)
        if not sel:
            out[(b, h, i)] = np.zeros((e - s, d))
            sums[(b, h, i)] = np.zeros(e - s, dtype=np.int64)
            continue
        keys = _keys_of(sel, bk, N)
        # per-key score scale c_j = fl32(fl32(sq_i sk_blk(j)) / sqrt(d))
        c = np.concatenate([np.full(block_range(j, bk, N)[1] - block_range(j, bk, N)[0],
                                    _F32(_F32(sq[b, h, i] * sk[b, h, j]) * lam), dtype=np.float32)
                            for j in sel])
        I = q8[b, h, s:e] @ k8[b, h, keys].T                   # exact integer scores
        S = (I.astype(np.float32) * c[None, :]).astype(np.float32)
        o = np.zeros((e - s, d))
        L = np.zeros(e - s, dtype=np.int64)
        for t in range(e - s):
            codes = p_codes(I[t], c, S[t].max())
            num = codes @ v8[b, h, keys]                       # exact integers
            L[t] = codes.sum()
            o[t] = sv[b, h].astype(np.float64) * num / float(L[t])
        out[(b, h, i)] = o
        sums[(b, h, i)] = L
    return (out, sums) if with_sums else out


# ------------------------- single-pass 8-bit sparse branch (E4M3 P and V)
# A second reading of [SLA2 §三]'s 8-bit sparse branch, taken in ONE pass over
# a row's keys: the scores come from the 8-bit integer codes of Q and K as in
# the two-pass branch above, while P and V are 8-bit floating-point numbers in
# the E4M3 format of the OCP 8-bit floating-point specification (1 sign bit, 4
# exponent bits with bias 7, 3 mantissa bits, no infinities, largest finite
# value 448, subnormals m * 2^-9 at exponent field 0).  A floating-point P has
# the headroom an online softmax needs (codes up to 256 with room to 448), so
# the row maximum need not be known before the first code is formed.
# * codes: Q per query block and K per key block as quantize_i8 (integers in
#   [-127, 127]); V per channel over the whole sequence of a head: code =
#   E4M3(fl32(x * fl32(448 / amax))), scale = fl32(amax / 448), E4M3()
#   rounding to the nearest value, ties to the even mantissa (zero codes and
#   scale when amax is 0);
# * scores I = q8 . k8 (exact integers), S = fl32(I c) with c = fl32(fl32(sq *
#   sk) * fl32(1 / sqrt(d))), as in the two-pass branch;
# * the row's selected keys in 64-key units, in the mask's order; m = the
#   largest S so far, the current unit's included; the unit's P codes are
#   E4M3(256 exp(S - m)) (at most 256); whenever m rises, what the earlier
#   units accumulated is multiplied by exp(m_old - m_new);
# * O = sv * (sum_u w_u sum_j code_j v8_j) / (sum_u w_u sum_j code_j), w_u =
#   exp(m_u - m_last); a row with no selected block gives 0.
# A P code is a quantised value decided by floating point, so it is decided in
# the precision the kernel computes it in (as the integer branch's codes are):
# 256 exp(S - m) is taken as fl32(2^t), t = fl32(I a - b), a = fl32(c log2 e),
# b = fl32(fl32(m log2 e) - 8) (f8_p_codes); tests pin that against the exact
# value.
_E4M3_MAX = 448.0
_F8_UNIT = 64      # keys per unit of the single pass


def e4m3(x) -> np.ndarray:
    """x (float64) rounded to the nearest E4M3 value, ties to the even
    mantissa.  |x| must not exceed 449 (the callers' values stay at or below
    448 up to float32 rounding); results above 448 become 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all(a <= 449.0), "value outside the E4M3 range"
    _, e = np.frexp(a)                       # a = f 2^e, f in [0.5, 1): binade 2^(e-1)
    e = np.maximum(e - 1, -6)                # exponent of the binade, subnormals at -6
    step = np.ldexp(1.0, (e - 3).astype(np.int64))  # spacing of 3 mantissa bits there
    r = np.rint(a / step) * step             # a / step is exact; rint: half to even
    return np.copysign(np.minimum(r, _E4M3_MAX), x)


def e4m3_decode(bits) -> np.ndarray:
    """Values of E4M3 bit patterns (uint8); the two NaN patterns give NaN."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    E, M = (b >> 3) & 0xF, b & 0x7
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 0xF) & (M == 0x7), np.nan, mag)
    return sign * mag


def _f8_codes(x32: np.ndarray, amax: np.float32) -> Tuple[np.ndarray, np.float32]:
    amax = _F32(amax)
    if amax == 0:
        return np.zeros(x32.shape), _F32(0.0)
    r = _F32(_F32(_E4M3_MAX) / amax)
    return e4m3((x32 * r).astype(np.float32).astype(np.float64)), _F32(amax / _F32(_E4M3_MAX))


def quantize_e4m3_channels(V) -> Tuple[np.ndarray, np.ndarray]:
    """Per-channel E4M3 codes (as float64 values) of V [B, H, N, d]: one scale
    per (b, h, d index) over all N rows.  Returns (codes [B, H, N, d], scales
    float32 [B, H, d])."""
    Vf = _as_f32_exact(V)
    B, H, N, d = Vf.shape
    codes, scales = np.zeros((B, H, N, d)), np.zeros((B, H, d), dtype=np.float32)
    for bb in range(B):
        for h in range(H):
            for c in range(d):
                col = Vf[bb, h, :, c]
                codes[bb, h, :, c], scales[bb, h, c] = _f8_codes(col, np.abs(col).max())
    return codes, scales


def quantize_i8f8(Q, K, V, bq: int, bk: int) -> Dict:
    """The single-pass branch's 8-bit inputs: Q per query block and K per key
    block as integers (quantize_blocks), V per channel as E4M3 values."""
    q8, sq = quantize_blocks(Q, bq)
    k8, sk = quantize_blocks(K, bk)
    v8, sv = quantize_e4m3_channels(V)
    return {"q8": q8, "sq": sq, "k8": k8, "sk": sk, "v8": v8, "sv": sv}


def f8_p_codes(R: np.ndarray, a, b) -> np.ndarray:
    """E4M3 P codes of raw scores R (float32 values: here the exact integer
    scores I, which float32 holds) with a = fl32(c log2 e) and
    b = fl32(fl32(m log2 e) - 8) (broadcast against R): E4M3(fl32(2^t)),
    t = fl32(R a - b) with the product and difference exact in float64 before
    the one rounding, 2^t taken in float64 and rounded to float32."""
    t = (R.astype(np.float64) * np.asarray(a, np.float64) - np.asarray(b, np.float64)).astype(np.float32)
    p = np.exp2(t.astype(np.float64)).astype(np.float32)
    return e4m3(p.astype(np.float64))


def sparse_branch_i8f8(qz: Dict, bq: int, bk: int, row_ptr, col_idx, rows=None, with_sums: bool = False):
    """The single-pass 8-bit sparse branch on quantize_i8f8's codes (see the
    section comment).  Returns {(b, h, i): [rows_in_block, d]} and with
    with_sums also {(b, h, i): (L, m, A)}: per query the weighted sum of P codes
    relative to the final maximum, that maximum (float32), and per output the
    same weighted mean of |v| (the scale of the float32 sums)."""
    q8, k8 = qz["q8"].astype(np.int64), qz["k8"].astype(np.int64)
    v8, sq, sk, sv = qz["v8"], qz["sq"], qz["sk"], qz["sv"]
    B, H, N, d = q8.shape
    Nq = n_blocks(N, bq)
    lam = _F32(1.0 / math.sqrt(d))
    out, sums = {}, {}
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = [int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]]]
        s, e = block_range(i, bq, N)
        n = e - s
        if not sel:
            out[(b, h, i)] = np.zeros((n, d))
            sums[(b, h, i)] = (np.zeros(n), np.full(n, -np.inf, dtype=np.float32), np.zeros((n, d)))
            continue
        # the row's keys block by block, each block cut into 64-key units
        units = []
        for j in sel:
            ks, ke = block_range(j, bk, N)
            c = _F32(_F32(sq[b, h, i] * sk[b, h, j]) * lam)
            for u0 in range(ks, ke, _F8_UNIT):
                units.append((np.arange(u0, min(u0 + _F8_UNIT, ke)), c))
        num, anum, L = np.zeros((n, d)), np.zeros((n, d)), np.zeros(n)
        m = np.full(n, -np.inf, dtype=np.float32)
        for keys, c in units:
            I = q8[b, h, s:e] @ k8[b, h, keys].T                      # exact integers
            S = (I.astype(np.float32) * c).astype(np.float32)
            mu = np.maximum(m, S.max(axis=1))
            w = np.where(np.isfinite(m), np.exp(m.astype(np.float64) - mu.astype(np.float64)), 0.0)
            num *= w[:, None]
            anum *= w[:, None]
            L *= w
            m = mu
            a = _F32(c * _LOG2E_F32)
            bb = ((m * _LOG2E_F32).astype(np.float32) - _F32(8.0)).astype(np.float32)
            p8 = f8_p_codes(I.astype(np.float32), a, bb[:, None])
            num += p8 @ v8[b, h, keys]
            anum += p8 @ np.abs(v8[b, h, keys])
            L += p8.sum(axis=1)
        svd = sv[b, h].astype(np.float64)[None, :]
        out[(b, h, i)] = svd * num / L[:, None]
        sums[(b, h, i)] = (L, m, svd * anum / L[:, None])
    return (out, sums) if with_sums else out


# -------------------------------------------------------- sparse backward
# The gradient of the sparse branch with the mask held fixed (the block
# selection is a discrete choice; the pages train through it with the
# selection fixed per step [SLA2 §四, stage 2 uses hard Top-k]).  Written as
# the derivative of the forward definition above, taken by torch's autograd
# in float64 on the CPU, one row block at a time; pinned by central finite
# differences and by the full-mask case (dense attention's gradient).
def sparse_branch_backward(Q, K, V, bq: int, bk: int, row_ptr, col_idx, dO, rows=None) -> Dict[str, np.ndarray]:
    """dQ, dK, dV of L = sum(O_s * dO), O_s the sparse branch of
    sparse_branch() (rows with no selected block contribute nothing), one row
    block at a time.  With `rows` (a list of (b, h, i)) only those row blocks
    are differentiated: their dQ rows are exact, dK and dV hold only their
    share."""
    import torch
    Qt, Kt, Vt = (torch.tensor(as_f64(x)) for x in (Q, K, V))
    G = torch.tensor(as_f64(dO))
    B, H, N, d = Qt.shape
    Nq = n_blocks(N, bq)
    dQ, dK, dV = torch.zeros_like(Qt), torch.zeros_like(Kt), torch.zeros_like(Vt)
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        if len(sel) == 0:
            continue
        keys = torch.tensor(_keys_of(sel, bk, N))
        s, e = block_range(i, bq, N)
        q = Qt[b, h, s:e].clone().requires_grad_(True)
        k = Kt[b, h, keys].clone().requires_grad_(True)
        v = Vt[b, h, keys].clone().requires_grad_(True)
        P = torch.softmax(q @ k.T / math.sqrt(d), dim=-1)
        o = P @ v
        (o * G[b, h, s:e]).sum().backward()
        dQ[b, h, s:e] += q.grad
        dK[b, h, keys] += k.grad
        dV[b, h, keys] += v.grad
    return {"dQ": dQ.numpy(), "dK": dK.numpy(), "dV": dV.numpy()}


def alpha_grad(dO, Os, Ol) -> np.ndarray:
    """d/d alpha_h of sum(O * dO) with O = alpha_h O_s + (1 - alpha_h) O_l
    [SLA2 §二]: sum over the head's tokens of dO . (O_s - O_l).  Returns [H]."""
    g = as_f64(dO) * (as_f64(Os) - as_f64(Ol))
    return g.sum(axis=(0, 2, 3))


# -------------------------------------------------------- linear backward
def linear_branch_backward(Q, K, V, bq: int, bk: int, row_ptr, col_idx, dO, rows=None) -> Dict[str, np.ndarray]:
    """dQ, dK, dV of L = sum(O_l * dO), O_l the linear branch of
    linear_branch() over each row block's unselected keys (mask fixed), as
    the derivative of that definition taken by torch's autograd in float64,
    one row block at a time (rows whose blocks are all selected contribute
    nothing).  With `rows` (a list of (b, h, i)) only those row blocks are
    differentiated: their dQ rows are exact, dK and dV hold only their share."""
    import torch
    Qt, Kt, Vt = (torch.tensor(as_f64(x)) for x in (Q, K, V))
    G = torch.tensor(as_f64(dO))
    B, H, N, d = Qt.shape
    Nq, Nk = n_blocks(N, bq), n_blocks(N, bk)
    dQ, dK, dV = torch.zeros_like(Qt), torch.zeros_like(Kt), torch.zeros_like(Vt)
    for (b, h, i) in _rows(B, H, Nq, rows):
        r = (b * H + h) * Nq + i
        sel = set(int(j) for j in col_idx[row_ptr[r]:row_ptr[r + 1]])
        unsel = [j for j in range(Nk) if j not in sel]
        if not unsel:
            continue
        keys = torch.tensor(_keys_of(unsel, bk, N))
        s, e = block_range(i, bq, N)
        q = Qt[b, h, s:e].clone().requires_grad_(True)
        k = Kt[b, h, keys].clone().requires_grad_(True)
        v = Vt[b, h, keys].clone().requires_grad_(True)
        fq = torch.nn.functional.elu(q) + 1.0
        fk = torch.nn.functional.elu(k) + 1.0
        A = fq @ fk.T
        o = (A @ v) / A.sum(dim=1, keepdim=True)
        (o * G[b, h, s:e]).sum().backward()
        dQ[b, h, s:e] += q.grad
        dK[b, h, keys] += k.grad
        dV[b, h, keys] += v.grad
    return {"dQ": dQ.numpy(), "dK": dK.numpy(), "dV": dV.numpy()}
