"""Seeded synthetic inputs for the KDA forward workloads.

This module is shared by the CPU oracle (``oracle/``), the tests and the
benchmark.  It holds random-number recipes, shapes and dtype conversion only:
none of the operator's arithmetic (gate, decay, recurrence) lives here.

Every workload follows the head geometry of the Kimi K3 KDA layer (96 heads,
d_k = d_v = 128, chunk 64; see "Kimi K3 模型结构（7）：结构决定系统",
section "公式 (17) 的推导" for the head count, and "序列维度（下）" for C = 64).

Recipe conventions (stated once, used everywhere):
  * RNG: ``numpy.random.default_rng(seed)`` (PCG64); float32 draws;
    draw order q, k, v, z, beta, A, S0, lengths, accepted, bonus.
  * "N(mu, s)" in a workload description means standard deviation s.
  * q and k are L2-normalised per (token, head) in float32 before casting.
  * beta = sigmoid(N(0,1)) is drawn here, since the operator takes beta in (0,1).
  * bf16 casts round to nearest even.  The oracle reads the very same bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D = 128          # d_k = d_v
CHUNK = 64       # C
G_MIN = -5.0     # lower bound of the per-step log-decay


# ----------------------------------------------------------------------------
# bf16 helpers (storage only: bf16 values are kept as uint16 bit patterns)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest even), returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A host array in the storage dtype the operator receives.

    ``data`` is float32 for dtype "f32" and uint16 bf16 bits for dtype "bf16".
    """
    data: np.ndarray
    dtype: str  # "f32" | "bf16"

    @property
    def shape(self):
        return self.data.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "f32":
            return self.data
        return bf16_bits_to_f32(self.data)

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        return Tensor(np.ascontiguousarray(x, dtype=np.float32), "f32")
    if dtype == "bf16":
        return Tensor(f32_to_bf16_bits(x), "bf16")
    raise ValueError(dtype)


def _l2norm_last(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid_f32(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float32)))).astype(np.float32)


# ----------------------------------------------------------------------------
# Prefill inputs
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    q: Tensor            # [T, H, D]
    k: Tensor            # [T, H, D]
    v: Tensor            # [T, H, D]
    z: Tensor            # [T, H, D]  gate logits
    beta: Tensor         # [T, H]
    A_log: np.ndarray    # [H] float32
    S0: Optional[np.ndarray]   # [N, H, D, D] float32 or None
    cu_seqlens: np.ndarray     # [N+1] int32
    g_min: float = G_MIN
    dtype: str = "bf16"
    gate: str = "bounded"      # "bounded" (g_min applies) or "softplus" (no lower bound)
    raw: bool = False          # q, k unnormalised and beta a logit (normalised in the operator)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)


def _draw_qkvzb(rng, T, H, d, dtype, z_mean=0.0, z_std=1.0, raw=False):
    """raw: q, k left unnormalised and beta left as its logit (the same draws)."""
    q = rng.standard_normal((T, H, d), dtype=np.float32)
    k = rng.standard_normal((T, H, d), dtype=np.float32)
    if not raw:
        q, k = _l2norm_last(q), _l2norm_last(k)
    v = rng.standard_normal((T, H, d), dtype=np.float32)
    z = rng.standard_normal((T, H, d), dtype=np.float32)
    if z_std != 1.0:
        z *= np.float32(z_std)
    if z_mean != 0.0:
        z += np.float32(z_mean)
    beta = rng.standard_normal((T, H), dtype=np.float32)
    if not raw:
        beta = _sigmoid_f32(beta)
    return (_store(q, dtype), _store(k, dtype), _store(v, dtype), _store(z, dtype),
            _store(beta, dtype))


def log_uniform_lengths(rng, total: int, lo: int, hi: int) -> np.ndarray:
    """Document lengths L = round(exp(U(ln lo, ln hi))) until ``total`` is reached.

    The last document is cut to the remainder; a remainder shorter than ``lo``
    is merged into the previous document.
    """
    lens = []
    acc = 0
    while acc < total:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = min(L, total - acc)
        lens.append(L)
        acc += L
    if len(lens) > 1 and lens[-1] < lo:
        last = lens.pop()
        lens[-1] += last
    return np.asarray(lens, dtype=np.int64)


def cu_from_lengths(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


def make_prefill(seed: int, T: int, H: int, dtype: str = "bf16", *, A_std: float = 0.5,
                 lengths=None, varlen_total: Optional[int] = None, varlen_lo: int = 64,
                 varlen_hi: int = 16384, s0_std: float = 0.0, s0_docs: str = "first",
                 z_mean: float = 0.0, z_std: float = 1.0, d: int = D,
                 gate: str = "bounded", raw: bool = False) -> PrefillInputs:
    """Generic prefill recipe.

    ``lengths`` gives explicit document lengths; ``varlen_total`` draws them
    log-uniformly; otherwise one document of length T.  ``s0_std > 0`` gives
    document 0 (``s0_docs="first"``) or every document (``"all"``) an initial
    state ~ N(0, s0_std); other documents start from zero.
    """
    rng = np.random.default_rng(seed)
    q, k, v, z, beta = _draw_qkvzb(rng, T, H, d, dtype, z_mean=z_mean, z_std=z_std, raw=raw)
    A_log = (rng.standard_normal(H, dtype=np.float32) * np.float32(A_std)).astype(np.float32) \
        if A_std > 0 else np.zeros(H, dtype=np.float32)
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int64)
    elif varlen_total is not None:
        assert varlen_total == T
        lens = None  # drawn after S0 to keep the draw order q,k,v,z,beta,A,S0,lengths
    else:
        lens = np.asarray([T], dtype=np.int64)
    S0 = None
    n_docs_for_s0 = None if lens is None else len(lens)
    if s0_std > 0:
        # The state for document 0 is drawn before the lengths; further documents
        # (``s0_docs="all"``) are drawn after them.
        S0_first = (rng.standard_normal((H, d, d), dtype=np.float32) * np.float32(s0_std))
    if lens is None:
        lens = log_uniform_lengths(rng, varlen_total, varlen_lo, varlen_hi)
        n_docs_for_s0 = len(lens)
    assert int(lens.sum()) == T, (lens.sum(), T)
    if s0_std > 0:
        S0 = np.zeros((n_docs_for_s0, H, d, d), dtype=np.float32)
        S0[0] = S0_first
        if s0_docs == "all" and n_docs_for_s0 > 1:
            S0[1:] = rng.standard_normal((n_docs_for_s0 - 1, H, d, d), dtype=np.float32) \
                * np.float32(s0_std)
    return PrefillInputs(q=q, k=k, v=v, z=z, beta=beta, A_log=A_log, S0=S0,
                         cu_seqlens=cu_from_lengths(lens), dtype=dtype, gate=gate, raw=raw)


# ----------------------------------------------------------------------------
# Decode / speculative-verify inputs
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeInputs:
    state: np.ndarray     # [N, H, D, D] float32 (saved state before the draft window)
    cq: Tensor            # [N, W, H, D] cached projected draft inputs
    ck: Tensor
    cv: Tensor
    cz: Tensor
    cbeta: Tensor         # [N, W, H]
    accepted: np.ndarray  # [N] int32 in 0..W
    nq: Tensor            # [N, H, D] bonus-token inputs
    nk: Tensor
    nv: Tensor
    nz: Tensor
    nbeta: Tensor         # [N, H]
    A_log: np.ndarray     # [H] float32
    W: int
    g_min: float = G_MIN
    dtype: str = "bf16"
    # drafts of the next window, run after the bonus token (outputs only)
    wq: Optional[Tensor] = None   # [N, W2, H, D]
    wk: Optional[Tensor] = None
    wv: Optional[Tensor] = None
    wz: Optional[Tensor] = None
    wbeta: Optional[Tensor] = None  # [N, W2, H]
    W2: int = 0
    raw: bool = False     # q, k unnormalised and beta a logit (normalised in the operator)
    gate: str = "bounded"  # "bounded" (g_min applies) or "softplus" (no lower bound)

    @property
    def N(self) -> int:
        return int(self.state.shape[0])

    @property
    def H(self) -> int:
        return int(self.state.shape[1])


def make_decode(seed: int, N: int, H: int, W: int = 4, dtype: str = "bf16", *,
                A_std: float = 0.5, s_std: float = 0.02, d: int = D,
                accepted=None, W2: int = 0, raw: bool = False,
                gate: str = "bounded") -> DecodeInputs:
    """Decode-with-verify recipe: draft cache first (q,k,v,z,beta order), then A,
    the saved state, the accepted lengths U{0..W}, then the bonus token, then (if
    W2 > 0) the W2 drafts of the next window.  The draws of a call with W2 > 0
    start with exactly those of the same call with W2 = 0.  ``gate`` names the
    gate the operator applies ("bounded" or "softplus"); it changes no draw."""
    rng = np.random.default_rng(seed)
    T = N * W
    q, k, v, z, beta = _draw_qkvzb(rng, T, H, d, dtype, raw=raw)
    cq = Tensor(q.data.reshape(N, W, H, d), dtype)
    ck = Tensor(k.data.reshape(N, W, H, d), dtype)
    cv = Tensor(v.data.reshape(N, W, H, d), dtype)
    cz = Tensor(z.data.reshape(N, W, H, d), dtype)
    cb = Tensor(beta.data.reshape(N, W, H), dtype)
    A_log = (rng.standard_normal(H, dtype=np.float32) * np.float32(A_std)).astype(np.float32) \
        if A_std > 0 else np.zeros(H, dtype=np.float32)
    state = rng.standard_normal((N, H, d, d), dtype=np.float32) * np.float32(s_std)
    if accepted is None:
        acc = rng.integers(0, W + 1, size=N).astype(np.int32)
    else:
        acc = np.asarray(accepted, dtype=np.int32)
        assert acc.shape == (N,)
    nq, nk, nv, nz, nb = _draw_qkvzb(rng, N, H, d, dtype, raw=raw)
    win = {}
    if W2 > 0:
        wq, wk, wv, wz, wb = _draw_qkvzb(rng, N * W2, H, d, dtype, raw=raw)
        win = dict(wq=Tensor(wq.data.reshape(N, W2, H, d), dtype),
                   wk=Tensor(wk.data.reshape(N, W2, H, d), dtype),
                   wv=Tensor(wv.data.reshape(N, W2, H, d), dtype),
                   wz=Tensor(wz.data.reshape(N, W2, H, d), dtype),
                   wbeta=Tensor(wb.data.reshape(N, W2, H), dtype), W2=W2)
    return DecodeInputs(state=state, cq=cq, ck=ck, cv=cv, cz=cz, cbeta=cb, accepted=acc,
                        nq=nq, nk=nk, nv=nv, nz=nz, nbeta=nb, A_log=A_log, W=W, dtype=dtype,
                        raw=raw, gate=gate, **win)


# ----------------------------------------------------------------------------
# The five named workloads
# ----------------------------------------------------------------------------
WORKLOADS = {
    0: "tiny fp32: H=2, T=256, A=0, S0=0",
    1: "single-sequence prefill bf16: H=96, T=8192",
    2: "long prefill, one TP rank: H=8, T=262144, one segment per CU",
    3: "packed varlen prefill bf16: 65536 tokens, H=96, log-uniform docs [64,16384]",
    4: "decode with speculative verify: N=512, H=96, W=4 drafts + bonus",
}


def workload(idx: int, *, scale_T: Optional[int] = None, scale_H: Optional[int] = None,
             scale_N: Optional[int] = None):
    """Inputs for workload ``idx`` (seed = idx).  The ``scale_*`` arguments shrink a
    workload for CPU-sized checks while keeping its recipe."""
    if idx == 0:
        return make_prefill(0, scale_T or 256, scale_H or 2, "f32", A_std=0.0)
    if idx == 1:
        return make_prefill(1, scale_T or 8192, scale_H or 96, "bf16", A_std=0.5)
    if idx == 2:
        return make_prefill(2, scale_T or 262144, scale_H or 8, "bf16", A_std=0.5)
    if idx == 3:
        T = scale_T or 65536
        return make_prefill(3, T, scale_H or 96, "bf16", A_std=0.5, varlen_total=T,
                            s0_std=0.02, s0_docs="first")
    if idx == 4:
        return make_decode(4, scale_N or 512, scale_H or 96, 4, "bf16")
    raise ValueError(idx)


# ----------------------------------------------------------------------------
# Moving inputs to a device (storage only)
# ----------------------------------------------------------------------------
def to_torch(t, device="cuda"):
    """kda_gen.Tensor (or float32 ndarray) -> torch tensor on ``device``.
    bf16 bit patterns become torch.bfloat16 without any rounding."""
    import torch
    if isinstance(t, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(t)).to(device)
    if t.dtype == "bf16":
        return torch.from_numpy(t.data.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(t.data).to(device)


def from_torch(x) -> np.ndarray:
    """torch tensor (bf16 or fp32) -> float64 numpy array with the exact values."""
    import torch
    x = x.detach().to("cpu")
    if x.dtype == torch.bfloat16:
        return bf16_bits_to_f32(x.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    return x.to(torch.float64).numpy()
