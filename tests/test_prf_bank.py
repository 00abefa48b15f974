"""Pins of the PRF bank preparation (chunked_causal_linear_k1_amd/prf_bank.py) against what
"Linearized 2-Simplicial Attention" (section 3.2 and appendix B.1) and the mathematics fix:
orthogonal rows within each block, chi_d radii, Haar-distributed directions (the sign fix),
an unbiased softmax-kernel estimate, and a lower variance than independent rows. CPU only."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from chunked_causal_linear_k1_amd import prf_bank


def test_rows_within_a_block_are_orthogonal():
    d, m = 16, 40  # two full blocks and a partial third
    w = prf_bank.orthogonal_bank(2, m, d, seed=1, dtype=torch.float64).numpy()
    for h in range(2):
        for b0 in range(0, m, d):
            blk = w[h, b0:b0 + d]
            g = blk @ blk.T
            off = g - np.diag(np.diag(g))
            assert np.abs(off).max() < 1e-10 * np.diag(g).max()


def test_radii_follow_chi_d():
    """Row norms are chi_d: mean sqrt(2) Gamma((d+1)/2) / Gamma(d/2), variance d - mean^2."""
    d, m, H = 8, 64, 64
    r = np.linalg.norm(prf_bank.orthogonal_bank(H, m, d, seed=2, dtype=torch.float64).numpy(), axis=-1).ravel()
    mean = math.sqrt(2.0) * math.exp(math.lgamma((d + 1) / 2) - math.lgamma(d / 2))
    var = d - mean ** 2
    se = math.sqrt(var / r.size)
    assert abs(r.mean() - mean) < 5 * se, (r.mean(), mean, se)
    assert abs(r.var() - var) < 0.1 * var


def test_directions_are_haar():
    """With columns of Q times sign(R_aa) the directions are Haar-distributed: the first entry
    of a block's first row is positive half the time. Without the fix the common Householder
    QR returns it non-positive every time."""
    d, H = 6, 1000
    w = prf_bank.orthogonal_bank(H, d, d, seed=3, dtype=torch.float64).numpy()
    frac = float((w[:, 0, 0] > 0).mean())
    assert abs(frac - 0.5) < 5 * math.sqrt(0.25 / H), frac
    # every entry of a Haar direction has mean 0 and variance 1/d
    dirs = w / np.linalg.norm(w, axis=-1, keepdims=True)
    assert abs(dirs.mean()) < 5 / math.sqrt(dirs.size * d)
    assert abs((dirs ** 2).mean() - 1.0 / d) < 1e-12


def test_unbiased_with_lower_variance_than_independent_rows():
    """E[psi(x) . psi(y)] = exp(x . y) for both banks (each row is marginally N(0, I)); the
    orthogonal bank's estimate varies less ("Linearized 2-Simplicial Attention", appendix B.1)."""
    d, n = 16, 3000
    rng = np.random.default_rng(4)
    x = rng.standard_normal(d) * 0.35
    y = rng.standard_normal(d) * 0.35
    target = math.exp(float(x @ y))

    def estimates(make):
        est = np.empty(n)
        for s in range(n):
            w = make(s)
            est[s] = float(oracle.feature(x, oracle.PSI_PRF, d, w) @ oracle.feature(y, oracle.PSI_PRF, d, w))
        return est

    orth = estimates(lambda s: prf_bank.orthogonal_bank(1, d, d, seed=10_000 + s, dtype=torch.float64)[0].numpy())
    iid = estimates(lambda s: prf_bank.gaussian_bank(1, d, d, seed=10_000 + s, dtype=torch.float64)[0].numpy())
    for est in (orth, iid):
        assert abs(est.mean() - target) < 5 * est.std(ddof=1) / math.sqrt(n), (est.mean(), target)
    assert orth.var() < 0.9 * iid.var(), (orth.var(), iid.var())
