"""Banks W for the positive random features psi(x)_p = exp(w_p . x - |x|^2/2) / sqrt(m).

The bank is a model parameter, drawn once and passed to lin_attn_prefill and
lin_attn_decode_step like q, k and v; this module only prepares it on the host.

- gaussian_bank: rows w_p ~ N(0, I_d) independently ("Linearized 2-Simplicial
  Attention", section 3.2).
- orthogonal_bank: the orthogonal Gaussian bank of the same page's appendix B.1. Each
  block of d rows is a Haar-distributed orthogonal matrix (QR of a Gaussian matrix with
  the columns of Q multiplied by the signs of R's diagonal), each row scaled by an
  independent chi_d radius, so every row is still marginally N(0, I_d) and the feature
  estimate stays unbiased, while rows within a block are orthogonal, which lowers its
  variance. Blocks are stacked until m rows are reached.

Both return [H, m, d] tensors, drawn in fp64 from a seeded generator and rounded once
to the requested dtype (bf16 by default: both the kernels and any reference then see
the same stored values).
"""
from __future__ import annotations

import numpy as np
import torch


def _haar_block(rng: np.random.Generator, d: int) -> np.ndarray:
    """d orthonormal rows, Haar-distributed: rows of Q^T for G = QR with sign(diag R) > 0."""
    g = rng.standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]  # column a times sign(R_aa)
    return q.T


def orthogonal_bank(H: int, m: int, d: int, seed: int = 0, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    out = np.empty((H, m, d), dtype=np.float64)
    for h in range(H):
        rows = []
        n = 0
        while n < m:
            dirs = _haar_block(rng, d)
            radii = np.sqrt(rng.chisquare(d, size=d))  # chi_d: the norm of a d-dim Gaussian
            rows.append(dirs * radii[:, None])
            n += d
        out[h] = np.concatenate(rows, axis=0)[:m]
    return torch.from_numpy(out).to(dtype)


def gaussian_bank(H: int, m: int, d: int, seed: int = 0, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal((H, m, d))).to(dtype)
