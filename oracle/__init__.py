"""CPU oracle for the Kimi Delta Attention forward (fp64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``linear_attention_fwd_amd``) and never imports it.

Contents
  * ``kda_oracle.c`` -- gate (eq. (5) of the "序列维度（下）" page, and the
    unbounded Kimi Linear gate of the same section) and the
    token-by-token recurrence (eq. (1) of the systems page, delta form of the
    SemiAnalysis page), fp64, OpenMP over (document, head).
  * ``brute.py``     -- NumPy explicit-matrix form for tiny inputs
    (M_t = (I - beta k k^T) Diag(alpha), segment pairs and their composition).
  * ``chunk_form.py``-- the chunkwise (UT-transform) form, fp64, used only to
    check that the chunked rewrite equals the recurrence.
  * ``l2_normalize``, ``sigmoid``, ``operands`` (below) -- for raw inputs, the
    q/k L2 normalisation and beta sigmoid that the operator then performs itself.

Pins: see ``tests/test_oracle_pins.py``.  Every oracle function is pinned by
at least one closed form, special case or independent formulation there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (IEEE semantics: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o",
           _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # KDA_ORACLE_LIB: another build of kda_oracle.c (the tests run the pins on a
    # sanitizer build this way)
    path = os.environ.get("KDA_ORACLE_LIB")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.kda_oracle_gate.argtypes = [dp, dp, ctypes.c_double, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, dp]
    lib.kda_oracle_gate.restype = None
    lib.kda_oracle_gate_softplus.argtypes = [dp, dp, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_int32, dp]
    lib.kda_oracle_gate_softplus.restype = None
    lib.kda_oracle_recurrent.argtypes = [dp, dp, dp, dp, dp, dp, ip, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, dp, dp,
                                         ctypes.c_int32]
    lib.kda_oracle_recurrent.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def gate(z: np.ndarray, A_log: Optional[np.ndarray], g_min: float) -> np.ndarray:
    """g = g_min * sigmoid(exp(A_h) * z) in fp64; z: [T, H, dk]."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, H, dk = z.shape
    A = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float64)
    g = np.empty_like(z)
    _load().kda_oracle_gate(_dptr(z), _dptr(A), float(g_min), T, H, dk, _dptr(g))
    return g


def gate_softplus(z: np.ndarray, A_log: Optional[np.ndarray]) -> np.ndarray:
    """Unbounded Kimi Linear gate g = -exp(A_h) * softplus(z) in fp64; z: [T, H, dk]."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    T, H, dk = z.shape
    A = None if A_log is None else np.ascontiguousarray(A_log, dtype=np.float64)
    g = np.empty_like(z)
    _load().kda_oracle_gate_softplus(_dptr(z), _dptr(A), T, H, dk, _dptr(g))
    return g


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """x / ||x||_2 over the last axis (the channels of one token and head), fp64; a
    zero vector stays zero.  The normalisation of q and k that the KDA kernels
    perform in-kernel when given unnormalised inputs ("序列维度（下）", section on
    which form each phase uses)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-x), fp64: beta from its logit (same section)."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def operands(inp, q: np.ndarray, k: np.ndarray, beta: np.ndarray):
    """(q, k, beta) as the recurrence takes them: unchanged, or, for inputs marked
    raw, q and k L2-normalised per (token, head) and beta = sigmoid(logit)."""
    if getattr(inp, "raw", False):
        return l2_normalize(q), l2_normalize(k), sigmoid(beta)
    return q, k, beta


def gate_of(inp, z: np.ndarray, heads=None) -> np.ndarray:
    """The gate that ``inp`` names ("bounded": equation (5); "softplus": the
    unbounded Kimi Linear map) on logits z [T, H', dk] of heads ``heads``."""
    A = inp.A_log if heads is None else inp.A_log[heads]
    if getattr(inp, "gate", "bounded") == "softplus":
        return gate_softplus(z, A)
    return gate(z, A, inp.g_min)


def recurrent(q, k, v, g, beta, S0=None, cu_seqlens=None, nthreads: int = 0):
    """Token recurrence on raw log-decays g (alpha = exp(g)).

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; S0: [N, H, dk, dv] or None;
    cu_seqlens: [N+1] or None (one document).  Returns (o [T,H,dv], S_final
    [N,H,dk,dv]) in fp64.
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is None:
        cu = np.asarray([0, T], dtype=np.int32)
    else:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    N = cu.shape[0] - 1
    assert cu[-1] == T
    if S0 is not None:
        S0 = np.ascontiguousarray(S0, dtype=np.float64)
        assert S0.shape == (N, H, dk, dv), S0.shape
    o = np.zeros((T, H, dv), dtype=np.float64)
    S_final = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_recurrent(
        _dptr(q), _dptr(k), _dptr(v), _dptr(g), _dptr(beta), _dptr(S0),
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), N, H, dk, dv, _dptr(o),
        _dptr(S_final), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_recurrent rejected its arguments")
    return o, S_final


def forward(inp, nthreads: int = 0):
    """Full operator on a ``kda_gen.PrefillInputs``: gate (and, for raw inputs, the
    q/k normalisation and beta sigmoid), then the recurrence."""
    g = gate_of(inp, inp.z.f64())
    S0 = None if inp.S0 is None else inp.S0.astype(np.float64)
    q, k, b = operands(inp, inp.q.f64(), inp.k.f64(), inp.beta.f64())
    return recurrent(q, k, inp.v.f64(), g, b, S0, inp.cu_seqlens, nthreads)


def decode(inp, nthreads: int = 0):
    """Speculative-verify replay on a ``kda_gen.DecodeInputs``.

    For each sequence n: start from the saved state, run its accepted[n] cached
    draft tokens, then the bonus token (the systems page, section "KDA：三种
    执行形态" on decode).  Returns (o of the bonus token [N,H,dv], state [N,H,dk,dv]).
    """
    N, W, H, d = inp.cq.shape
    acc = np.clip(inp.accepted.astype(np.int64), 0, W)
    lens = acc + 1
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    cq, ck, cv, cz = inp.cq.f64(), inp.ck.f64(), inp.cv.f64(), inp.cz.f64()
    cb = inp.cbeta.f64()
    q = np.empty((T, H, d)); k = np.empty((T, H, d)); v = np.empty((T, H, d))
    z = np.empty((T, H, d)); b = np.empty((T, H))
    nq, nk, nv, nz, nb = inp.nq.f64(), inp.nk.f64(), inp.nv.f64(), inp.nz.f64(), inp.nbeta.f64()
    for n in range(N):
        s, a = int(cu[n]), int(acc[n])
        q[s:s + a], k[s:s + a], v[s:s + a], z[s:s + a], b[s:s + a] = (
            cq[n, :a], ck[n, :a], cv[n, :a], cz[n, :a], cb[n, :a])
        q[s + a], k[s + a], v[s + a], z[s + a], b[s + a] = nq[n], nk[n], nv[n], nz[n], nb[n]
    g = gate_of(inp, z)
    q, k, b = operands(inp, q, k, b)
    o, S = recurrent(q, k, v, g, b, inp.state.astype(np.float64), cu, nthreads)
    o_bonus = o[cu[1:] - 1]
    return o_bonus, S


def decode_window(inp, nthreads: int = 0):
    """Decode step followed by the next draft window, on a ``kda_gen.DecodeInputs``
    with W2 > 0 (the systems page, section "KDA：三种执行形态" on decode: replay,
    bonus token and the next drafts in one loop).

    The tokens of sequence n are its accepted drafts, the bonus token, then its W2
    window drafts, run by the recurrence from the saved state.  Returns (o of the
    bonus token [N,H,dv], o of the window drafts [N,W2,H,dv], the state after the
    bonus token [N,H,dk,dv], the one that is kept: the window's drafts are not yet
    verified)."""
    N, W, H, d = inp.cq.shape
    W2 = inp.W2
    acc = np.clip(inp.accepted.astype(np.int64), 0, W)
    lens = acc + 1 + W2
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = np.empty((T, H, d)); k = np.empty((T, H, d)); v = np.empty((T, H, d))
    z = np.empty((T, H, d)); b = np.empty((T, H))
    parts = [(inp.cq.f64(), inp.ck.f64(), inp.cv.f64(), inp.cz.f64(), inp.cbeta.f64()),
             (inp.nq.f64()[:, None], inp.nk.f64()[:, None], inp.nv.f64()[:, None],
              inp.nz.f64()[:, None], inp.nbeta.f64()[:, None]),
             (inp.wq.f64(), inp.wk.f64(), inp.wv.f64(), inp.wz.f64(), inp.wbeta.f64())]
    for n in range(N):
        s = int(cu[n])
        for (pq, pk, pv, pz, pb), m in zip(parts, (int(acc[n]), 1, W2)):
            q[s:s + m], k[s:s + m], v[s:s + m], z[s:s + m], b[s:s + m] = (
                pq[n, :m], pk[n, :m], pv[n, :m], pz[n, :m], pb[n, :m])
            s += m
    g = gate_of(inp, z)
    q, k, b = operands(inp, q, k, b)
    o, _ = recurrent(q, k, v, g, b, inp.state.astype(np.float64), cu, nthreads)
    o_bonus = o[cu[:-1] + acc]
    o_window = np.stack([o[cu[n] + acc[n] + 1:cu[n + 1]] for n in range(N)])
    _, S = decode(inp, nthreads)
    return o_bonus, o_window, S
