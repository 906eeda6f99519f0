"""Seeded synthetic inputs shaped like video-DiT attention.

This module only draws and casts numbers.  It holds none of the attention
method's arithmetic and is shared by the tests, the benchmark and the oracle
harness, so that both sides of every parity check see the same inputs.

Recipe (one workload = one entry of ``WORKLOADS``):

* tokens sit on a (t, h, w) grid, flattened t-major: n = t*(Hh*W) + h*W + w;
* a d-dim sinusoid s(x)[2i] = sin(x * 10000^(-2i/d)), s(x)[2i+1] = cos(...),
  and the positional term PE(t, h, w) = s(t) + s(h) + s(w);
* Q = tau * (N(0,1) + 2*PE), K = N(0,1) + 2*PE, V = N(0,1);
* one ``numpy.random.default_rng(seed)`` stream (PCG64), drawn in this order:
  for b, for h: Q noise, K noise, V; then the per-head mixing ratio alpha;
  then the router matrices Wq, Wk ~ N(0, 1/d) (variance 1/d);
* everything is generated in float64 and rounded to the workload dtype with
  round-to-nearest-even (torch's CPU cast).

The positional term makes pooled query/key blocks that are near each other on
the grid score highly, which is what gives the pooled score maps the
concentrated-but-local structure of video attention.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    grid: Tuple[int, int, int]
    d: int
    bq: int
    bk: int
    k_frac: float
    p: float
    dtype: str                      # "fp32" or "bf16"
    alpha: Tuple[float, ...] = ()   # constant per-head alpha (empty: drawn)
    alpha_range: Tuple[float, float] = (0.6, 0.95)
    tau: float = 1.0
    router: bool = False
    seed: int = 0

    @property
    def N(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def Nq(self) -> int:
        return -(-self.N // self.bq)

    @property
    def Nk(self) -> int:
        return -(-self.N // self.bk)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Five workload families.  The grids 21x30x52 and 21x45x80 are the latent token
# grids of 480p and 720p video generation; H and d are the head layout of the
# 1.3B- and 14B-parameter video DiTs.
WORKLOADS = {
    # tiny fp32 case the oracle finishes in well under a second
    "tiny-fp32-N1024": Workload("tiny-fp32-N1024", B=1, H=2, grid=(4, 16, 16), d=64,
                                bq=64, bk=64, k_frac=0.1, p=0.6, dtype="fp32",
                                alpha=(1.0, 1.0), seed=1),
    # bf16 mask + sparse branch only (alpha = 1), about 90% block sparsity
    "video480p-sparse-N32760": Workload("video480p-sparse-N32760", B=1, H=12, grid=(21, 30, 52),
                                        d=128, bq=128, bk=64, k_frac=0.05, p=0.9,
                                        dtype="bf16", alpha=(1.0,) * 12, seed=2),
    # bf16 full sparse + linear forward at about 97% block sparsity
    "video480p-sla2-N32760": Workload("video480p-sla2-N32760", B=1, H=12, grid=(21, 30, 52),
                                      d=128, bq=128, bk=64, k_frac=0.03, p=0.5,
                                      dtype="bf16", alpha_range=(0.6, 0.95), seed=3),
    # bf16 720p-sized case, 40 heads
    "video720p-sla2-N75600": Workload("video720p-sla2-N75600", B=1, H=40, grid=(21, 45, 80),
                                      d=128, bq=128, bk=64, k_frac=0.04, p=0.7,
                                      dtype="bf16", alpha_range=(0.6, 0.95), seed=4),
    # learned-router sweep: tau in {0.25, 1, 4} x p in {0.3, 0.6, 0.9}
    "video480p-router-N32760": Workload("video480p-router-N32760", B=2, H=16, grid=(21, 30, 52),
                                        d=128, bq=128, bk=64, k_frac=0.03, p=0.6,
                                        dtype="bf16", alpha_range=(0.5, 0.95), router=True,
                                        seed=5),
}

ROUTER_TAUS = (0.25, 1.0, 4.0)
ROUTER_PS = (0.3, 0.6, 0.9)


def sinusoid(x: np.ndarray, d: int) -> np.ndarray:
    """d-dim sinusoidal encoding of integer positions x -> [len(x), d]."""
    i = np.arange(d // 2, dtype=np.float64)
    freq = np.power(10000.0, -2.0 * i / d)
    ang = np.asarray(x, dtype=np.float64)[:, None] * freq[None, :]
    out = np.empty((len(x), d), dtype=np.float64)
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang)
    return out


def positional(grid: Sequence[int], d: int) -> np.ndarray:
    """PE[n] = s(t) + s(h) + s(w) for tokens flattened t-major -> [N, d] float64."""
    T, Hh, W = grid
    st, sh, sw = sinusoid(np.arange(T), d), sinusoid(np.arange(Hh), d), sinusoid(np.arange(W), d)
    pe = st[:, None, None, :] + sh[None, :, None, :] + sw[None, None, :, :]
    return pe.reshape(T * Hh * W, d)


def torch_dtype(name: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(x).to(torch_dtype(dtype))


@dataclasses.dataclass
class Inputs:
    """Host tensors in the workload dtype (Q, K, V: [B, H, N, d]); alpha fp32 [H];
    Wq, Wk fp32 [d, d] or None."""
    wl: Workload
    Q: torch.Tensor
    K: torch.Tensor
    V: torch.Tensor
    alpha: torch.Tensor
    Wq: Optional[torch.Tensor]
    Wk: Optional[torch.Tensor]


def make(wl: Workload, seed: Optional[int] = None, heads: Optional[int] = None,
         N: Optional[int] = None) -> Inputs:
    """Draw one workload's inputs.

    ``heads`` limits generation to the first few heads of batch 0 (the draws of
    those heads are identical to the full run's); ``N`` overrides the token
    count (tokens are then taken from a flattened grid padded as needed), which
    is how ragged sizes such as N=1000 or 1001 are produced.
    """
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    n_tok = wl.N if N is None else int(N)
    T, Hh, W = wl.grid
    if n_tok <= T * Hh * W:
        pe = positional(wl.grid, wl.d)[:n_tok]
    else:  # extend along t
        t_needed = -(-n_tok // (Hh * W))
        pe = positional((t_needed, Hh, W), wl.d)[:n_tok]
    B = wl.B if heads is None else 1
    H = wl.H if heads is None else int(heads)
    tdt = torch_dtype(wl.dtype)
    Q = torch.empty((B, H, n_tok, wl.d), dtype=tdt)
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    for b in range(B):
        for h in range(H):
            qn = rng.standard_normal((n_tok, wl.d))
            kn = rng.standard_normal((n_tok, wl.d))
            vn = rng.standard_normal((n_tok, wl.d))
            Q[b, h] = _cast(wl.tau * (qn + 2.0 * pe), wl.dtype)
            K[b, h] = _cast(kn + 2.0 * pe, wl.dtype)
            V[b, h] = _cast(vn, wl.dtype)
    if wl.alpha:
        alpha = torch.tensor(list(wl.alpha)[:H], dtype=torch.float32)
        if alpha.numel() < H:
            alpha = torch.full((H,), float(wl.alpha[0]), dtype=torch.float32)
    else:
        lo, hi = wl.alpha_range
        alpha = torch.from_numpy(rng.uniform(lo, hi, size=wl.H)[:H]).to(torch.float32)
    Wq = Wk = None
    if wl.router:
        std = 1.0 / math.sqrt(wl.d)
        Wq = torch.from_numpy(rng.standard_normal((wl.d, wl.d)) * std).to(torch.float32)
        Wk = torch.from_numpy(rng.standard_normal((wl.d, wl.d)) * std).to(torch.float32)
    return Inputs(wl, Q, K, V, alpha, Wq, Wk)


def random_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
               scale: float = 1.0, with_pe: bool = True) -> Tuple[torch.Tensor, ...]:
    """Small ad-hoc inputs for edge-case tests: positional structure on a 1-D
    token line (t=1, h=1, w=N) plus noise."""
    rng = np.random.default_rng(seed)
    pe = sinusoid(np.arange(N), d) if with_pe else np.zeros((N, d))
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, H, N, d))
        out.append(x)
    q = scale * (out[0] + 2.0 * pe)
    k = out[1] + 2.0 * pe
    return _cast(q, dtype), _cast(k, dtype), _cast(out[2], dtype)
