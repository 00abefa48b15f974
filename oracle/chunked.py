"""fp64 statement of the chunked method itself -- TEST INFRASTRUCTURE ONLY.

Used to pin that "chunk summaries + exclusive scan + output pass" reproduces the
token-by-token recurrence (the claim that the scan is mathematically identical
to sequential accumulation: "Log-Depth Chunked Linear-Attention Scan",
Implementation notes). It follows that page's three kernels in order, extended
with the decay of "Linear Attention and Retentive Networks" (chunkwise recurrent
representation C), whose decay vectors Xi and Theta the page leaves undefined;
they are read off the recurrence as

  Theta_j = gamma^(j+1)         (prefix state seen by the j-th token of a chunk, 0-based)
  Xi_i    = gamma^(len-1-i)     (weight of token i in the chunk summary)
  D_ji    = gamma^(j-i), i <= j (intra-chunk decay), chunk decay a = gamma^len.

Summaries combine under the (non-commutative) monoid
  (a1, S1, Z1) (+) (a2, S2, Z2) = (a1 a2, a2 S1 + S2, a2 Z1 + Z2),  identity (1, 0, 0),
which is the additive monoid of the chunked-scan page when gamma = 1.
Padded positions of the last chunk contribute nothing (identity elements), as
that page requires ("padded positions must contribute zero summaries").
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .brute import feature_np


@dataclass
class Summary:
    a: float
    S: np.ndarray
    Z: np.ndarray


def combine(x: Summary, y: Summary) -> Summary:
    """x (+) y with x the earlier segment."""
    return Summary(x.a * y.a, y.a * x.S + y.S, y.a * x.Z + y.Z)


def identity(n_psi: int, d_v: int) -> Summary:
    return Summary(1.0, np.zeros((n_psi, d_v)), np.zeros(n_psi))


def scan_sequential(xs: List[Summary]) -> Tuple[List[Summary], int]:
    out, acc = [], identity(*xs[0].S.shape)
    for x in xs:
        out.append(acc)
        acc = combine(acc, x)
    return out, len(xs)


def scan_hillis_steele(xs: List[Summary]) -> Tuple[List[Summary], int]:
    """Inclusive Hillis-Steele scan in ceil(log2 n) rounds, shifted to exclusive."""
    n = len(xs)
    cur = list(xs)
    rounds, d = 0, 1
    while d < n:
        cur = [cur[i] if i < d else combine(cur[i - d], cur[i]) for i in range(n)]
        d *= 2
        rounds += 1
    return [identity(*xs[0].S.shape)] + cur[:-1], rounds


def scan_blelloch(xs: List[Summary]) -> Tuple[List[Summary], int]:
    """Work-efficient exclusive scan: up-sweep then down-sweep on a power-of-two tree.

    The down-sweep gives the left child the parent's prefix and the right child
    (parent prefix) (+) (left subtree sum); with a non-commutative monoid this order
    is what makes the result equal to the sequential prefix.
    """
    n = len(xs)
    shape = xs[0].S.shape
    n2 = 1
    while n2 < n:
        n2 *= 2
    x = list(xs) + [identity(*shape) for _ in range(n2 - n)]
    levels = int(math.log2(n2)) if n2 > 1 else 0
    for d in range(levels):
        step = 2 ** (d + 1)
        for i in range(0, n2, step):
            x[i + step - 1] = combine(x[i + step // 2 - 1], x[i + step - 1])
    x[n2 - 1] = identity(*shape)
    for d in reversed(range(levels)):
        step = 2 ** (d + 1)
        for i in range(0, n2, step):
            left = x[i + step // 2 - 1]
            x[i + step // 2 - 1] = x[i + step - 1]
            x[i + step - 1] = combine(x[i + step - 1], left)
    return x[:n], 2 * levels


SCANS = {"sequential": scan_sequential, "hillis_steele": scan_hillis_steele, "blelloch": scan_blelloch}


def chunked(q: np.ndarray, k: np.ndarray, v: np.ndarray, psi: int, C: int, gamma: float = 1.0,
            normalize: int = 1, eps: float = 1e-6, w: np.ndarray | None = None,
            scan: str = "blelloch", S0: np.ndarray | None = None, Z0: np.ndarray | None = None,
            return_info: bool = False):
    """One (batch, head): q, k [T, d_k], v [T, d_v] fp64 -> o [T, d_v] (and final state)."""
    T, d_v = q.shape[0], v.shape[1]
    NC = -(-T // C)
    Tp = NC * C
    fq = feature_np(q, psi, w)
    fk = feature_np(k, 2 if psi == 3 else psi, w)  # keys never take the query-row shift
    n_psi = fq.shape[1]
    # right-pad to a whole number of chunks; padded keys are zeroed after the feature map
    fq_p = np.zeros((Tp, n_psi)); fq_p[:T] = fq
    fk_p = np.zeros((Tp, n_psi)); fk_p[:T] = fk
    v_p = np.zeros((Tp, d_v)); v_p[:T] = v
    g = float(gamma)
    j = np.arange(C)
    lag = j[:, None] - j[None, :]
    Dm = np.where(lag >= 0, np.power(g, np.maximum(lag, 0).astype(np.float64)), 0.0)
    theta = np.power(g, (j + 1).astype(np.float64))
    # Kernel 1: local outputs and chunk summaries
    num_loc, den_loc, sums = [], [], []
    for c in range(NC):
        sl = slice(c * C, (c + 1) * C)
        L = min(C, T - c * C)
        Qc, Kc, Vc = fq_p[sl], fk_p[sl], v_p[sl]
        A = (Qc @ Kc.T) * Dm
        num_loc.append(A @ Vc)
        den_loc.append(A.sum(axis=1))
        xi = np.zeros(C)
        xi[:L] = np.power(g, (L - 1 - np.arange(L)).astype(np.float64))
        Kx = Kc * xi[:, None]
        sums.append(Summary(g ** L, Kx.T @ Vc, Kx.sum(axis=0)))
    # Kernel 2: exclusive scan over chunk summaries
    prefix, rounds = SCANS[scan](sums)
    if S0 is not None:
        init = Summary(1.0, np.asarray(S0, dtype=np.float64),
                       np.zeros(n_psi) if Z0 is None else np.asarray(Z0, dtype=np.float64))
        prefix = [combine(init, p) for p in prefix]
    # Kernel 3: prefix broadcast + local term + normalisation
    o = np.zeros((T, d_v))
    for c in range(NC):
        L = min(C, T - c * C)
        Qc = fq_p[c * C:(c + 1) * C]
        num = theta[:, None] * (Qc @ prefix[c].S) + num_loc[c]
        den = theta * (Qc @ prefix[c].Z) + den_loc[c]
        out = num / (den + eps)[:, None] if normalize else num
        o[c * C:c * C + L] = out[:L]
    if not return_info:
        return o
    final = combine(prefix[-1], sums[-1])
    return o, {"rounds": rounds, "S": final.S, "Z": final.Z, "n_chunks": NC}
