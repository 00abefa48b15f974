"""Masked quadratic ("parallel") form of causal linear attention in numpy fp64.

TEST INFRASTRUCTURE ONLY: a second, independent definition used to pin the
recurrence oracle on tiny inputs. It never touches the HIP library.

  o = ((psi(Q) psi(K)^T) (.) D) V  /  (((psi(Q) psi(K)^T) (.) D) 1 + eps)

 * D_{n,m} = gamma^{n-m} for n >= m, else 0 ("Linear Attention and Retentive
   Networks", Multi-Scale Decay Formulation; parallel representation (A) is
   ((Q K^T) (.) D) V);
 * without decay the ratio is the causal linear-attention output of the same
   page ("The Associative Property and Linear Kernel Formulation", the
   sum over j = 1..i of phi(q_i) phi(k_j)^T v_j over the same sum without v_j).
 * An initial state (S0, Z0) enters as an extra term gamma^t psi(q_t) S0 for the
   t-th token (1-based), which is what the recurrence leaves of S0 after t steps.
"""
from __future__ import annotations

import numpy as np


def feature_np(x: np.ndarray, psi: int, w: np.ndarray | None = None) -> np.ndarray:
    """psi over the last axis of x [..., d_k] (fp64)."""
    if psi == 0:
        return x.copy()
    if psi == 1:
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    if psi in (2, 3):
        m = w.shape[0]
        lin = x @ w.T  # [..., m]
        half_sq = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
        logf = lin - half_sq
        if psi == 3:  # query-row shift: the row's largest log-feature becomes 0
            logf = logf - logf.max(axis=-1, keepdims=True)
        return np.exp(logf) / np.sqrt(m)
    raise ValueError(psi)


def quadratic(q: np.ndarray, k: np.ndarray, v: np.ndarray, psi: int, gamma: float = 1.0,
              normalize: int = 1, eps: float = 1e-6, w: np.ndarray | None = None,
              S0: np.ndarray | None = None, Z0: np.ndarray | None = None) -> np.ndarray:
    """One (batch, head): q, k [T, d_k], v [T, d_v] fp64 -> o [T, d_v] fp64."""
    T = q.shape[0]
    fq = feature_np(q, psi, w)
    fk = feature_np(k, 2 if psi == 3 else psi, w)  # keys never take the query-row shift
    A = fq @ fk.T  # [T, T], A[t, i] = psi(q_t) . psi(k_i)
    t_idx = np.arange(T)[:, None]
    i_idx = np.arange(T)[None, :]
    lag = t_idx - i_idx
    D = np.where(lag >= 0, np.power(float(gamma), np.maximum(lag, 0).astype(np.float64)), 0.0)
    A = A * D
    num = A @ v
    den = A.sum(axis=1)
    if S0 is not None:
        decay0 = np.power(float(gamma), np.arange(1, T + 1, dtype=np.float64))[:, None]
        num = num + decay0 * (fq @ S0)
        if Z0 is not None:
            den = den + decay0[:, 0] * (fq @ Z0)
    if not normalize:
        return num
    return num / (den + eps)[:, None]


def quadratic_gated(q: np.ndarray, k: np.ndarray, v: np.ndarray, psi: int, log_gate: np.ndarray,
                    normalize: int = 1, eps: float = 1e-6, w: np.ndarray | None = None,
                    S0: np.ndarray | None = None, Z0: np.ndarray | None = None) -> np.ndarray:
    """One (batch, head) with per-token, per-feature forget gates alpha_t = exp(log_gate_t)
    [T, n_psi], in the parallel form: with G_t = sum_{s <= t} log_gate_s,
        A[t, i] = sum_p psi(q_t)_p psi(k_i)_p exp(G_t[p] - G_i[p])    (i <= t)
        num_t   = sum_i A[t, i] v_i + sum_p psi(q_t)_p exp(G_t[p]) S0[p, :]
        den_t   = sum_i A[t, i]     + sum_p psi(q_t)_p exp(G_t[p]) Z0[p]
    ("Linear Attention and Retentive Networks", Data-Dependent Gating Mechanism: the product
    of the gates between token i and t scales what token i wrote)."""
    T = q.shape[0]
    fq = feature_np(q, psi, w)
    fk = feature_np(k, 2 if psi == 3 else psi, w)
    G = np.cumsum(np.asarray(log_gate, dtype=np.float64), axis=0)  # [T, n_psi]
    A = np.zeros((T, T))
    for t in range(T):
        dec = np.exp(G[t][None, :] - G[: t + 1])  # [t+1, n_psi]
        A[t, : t + 1] = (fk[: t + 1] * dec) @ fq[t]
    num = A @ v
    den = A.sum(axis=1)
    if S0 is not None:
        fqd = fq * np.exp(G)
        num = num + fqd @ S0
        if Z0 is not None:
            den = den + fqd @ Z0
    if not normalize:
        return num
    return num / (den + eps)[:, None]
