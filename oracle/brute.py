"""Explicit-matrix (brute force) form of the KDA recurrence, NumPy fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Meant for tiny inputs
(T <= 64): every token builds its d_k x d_k transition matrix.

  * ``transition``    -- M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), equation (1)
    of the systems page "Kimi K3 模型结构（7）", section "KDA 上下文并行".
  * ``run``           -- S_t = M_t S_{t-1} + beta_t k_t v_t^T, o_t = S_t^T q_t.
  * ``segment_pair``  -- (M, S~) of a token range: M = M_t ... M_1 (ordered
    product) and S~ the state reached from S = 0, equation (17) and step 1 of
    section "公式 (17) 的推导" on the same page.
  * ``compose``       -- (M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2), step 2 there.
"""
from __future__ import annotations

import numpy as np


def transition(k_t: np.ndarray, g_t: np.ndarray, beta_t: float) -> np.ndarray:
    dk = k_t.shape[0]
    return (np.eye(dk) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.exp(g_t))


def run(q, k, v, g, beta, S0=None):
    """Single head.  q, k, g: [T, dk]; v: [T, dv]; beta: [T].  Returns (o, S_T)."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S = transition(k[t], g[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def segment_pair(k, v, g, beta):
    """(M, S~) for the tokens given (single head)."""
    T, dk = k.shape
    dv = v.shape[1]
    M = np.eye(dk)
    S = np.zeros((dk, dv))
    for t in range(T):
        Mt = transition(k[t], g[t], beta[t])
        M = Mt @ M
        S = Mt @ S + beta[t] * np.outer(k[t], v[t])
    return M, S


def compose(p2, p1):
    """(M2, S2) o (M1, S1): apply segment 1 first, then segment 2."""
    M2, S2 = p2
    M1, S1 = p1
    return M2 @ M1, M2 @ S1 + S2


def apply_pair(p, S):
    M, St = p
    return M @ S + St
