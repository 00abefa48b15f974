"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the method: it draws Gaussian tensors with a
seeded ``torch.Generator``, scales them, rounds them once to the storage dtype
(round-to-nearest-even), and derives the per-head decay constants. Both sides of
every parity check read the very tensors produced here.

Recipe (also stated in the design notes):
  * generator: ``torch.Generator(device).manual_seed(seed)``; draw order q, k, v,
    then the PRF bank; values drawn as fp32 ``randn``, multiplied by the fp32
    scale, then cast to the storage dtype.
  * PRF bank: one W_h ~ N(0,1)^{n_psi x d_k} per head, shared across the batch,
    rounded to the storage dtype once ("Linearized 2-Simplicial Attention",
    section 3.2: the rows of the bank are standard Gaussian).
  * decay "retnet_spread": gamma_h = 1 - 2^(-5 - 5h/(H-1)), evaluated in fp64
    and rounded to fp32 ("Linear Attention and Retentive Networks", Multi-Scale
    Decay Formulation, which gives gamma = 1 - 2^(-5-h) per head; here the
    exponent is spread over the H heads).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch

from .workloads import DecodeWorkload, Workload, PSI_PRF, PSI_PRF_QSHIFT

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def gammas(w: Workload) -> Optional[np.ndarray]:
    """Per-head decay as fp32, or None for no decay (gamma = 1 exactly)."""
    if w.decay == "none":
        return None
    if w.decay == "retnet_spread":
        H = w.H
        g = [1.0 - 2.0 ** (-5.0 - (5.0 * h / (H - 1) if H > 1 else 0.0)) for h in range(H)]
        return np.asarray(g, dtype=np.float64).astype(np.float32)
    if w.decay.startswith("const:"):
        return np.full(w.H, float(w.decay.split(":", 1)[1]), dtype=np.float32)
    raise ValueError(f"unknown decay spec {w.decay!r}")


def _randn(shape, gen: torch.Generator, device, scale: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(torch.tensor(scale, dtype=torch.float32, device=device))
    return x.to(dtype)


def make_prefill_inputs(w: Workload, device: str = "cpu", seed: Optional[int] = None) -> Dict[str, object]:
    """q, k, v ([B,H,T,d], storage dtype), optional PRF bank [H,n_psi,d_k], gamma (fp32 numpy or None)."""
    s = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(s)
    dt = torch_dtype(w.dtype)
    q = _randn((w.B, w.H, w.T, w.d_k), gen, device, w.qk_scale, dt)
    k = _randn((w.B, w.H, w.T, w.d_k), gen, device, w.qk_scale, dt)
    v = _randn((w.B, w.H, w.T, w.d_v), gen, device, w.v_scale, dt)
    prf_w = None
    if w.psi in (PSI_PRF, PSI_PRF_QSHIFT):
        prf_w = _randn((w.H, w.n_psi, w.d_k), gen, device, 1.0, dt)
    return {"q": q, "k": k, "v": v, "prf_w": prf_w, "gamma": gammas(w)}


def make_log_gates(shape, seed: int, temp: float = 16.0, device: str = "cpu") -> torch.Tensor:
    """fp32 log forget gates logsigmoid(z) / temp with z ~ N(0, 1): the gate form of gated linear
    attention (a sigmoid of a projection, sharpened by a temperature), all in (-inf, 0)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return torch.nn.functional.logsigmoid(z) / temp


def make_upstream_grad(shape, seed: int, device: str = "cpu", dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """dL/do for a backward pass: N(0, 1) drawn in fp32 from a seeded generator, then stored in dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)


def varlen_lengths(w) -> List[int]:
    """The sequence lengths of a VarlenWorkload: uniform in [len_min, len_max], seeded."""
    rng = np.random.default_rng(w.seed)
    return [int(x) for x in rng.integers(w.len_min, w.len_max + 1, size=w.N)]


def make_varlen_inputs(w, device: str = "cpu") -> Dict[str, object]:
    """Packed q, k, v [total, H, d] of a VarlenWorkload, cu_seqlens (int32 [N + 1], on device),
    the lengths, the longest length and gamma (fp32 numpy or None)."""
    lengths = varlen_lengths(w)
    total = int(sum(lengths))
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 1)
    dt = torch_dtype(w.dtype)
    q = _randn((total, w.H, w.d_k), gen, device, w.qk_scale, dt)
    k = _randn((total, w.H, w.d_k), gen, device, w.qk_scale, dt)
    v = _randn((total, w.H, w.d_v), gen, device, w.v_scale, dt)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=device)
    return {"q": q, "k": k, "v": v, "prf_w": None, "gamma": gammas(w), "cu_seqlens": cu, "lengths": lengths,
            "max_len": max(lengths)}


def make_decode_prefix(w: DecodeWorkload, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """The seeded prefix whose keys/values fill the decode state: k, v [N,H,P,d] bf16."""
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    dt = torch_dtype(w.dtype)
    k = _randn((w.N, w.H, w.prefix_len, w.d_k), gen, device, 1.0, dt)
    v = _randn((w.N, w.H, w.prefix_len, w.d_v), gen, device, 1.0, dt)
    return {"k": k, "v": v}


def make_decode_steps(w: DecodeWorkload, steps: Optional[int] = None, device: str = "cpu") -> Dict[str, torch.Tensor]:
    """Per-step single-token inputs q, k, v [steps, N, H, d] bf16 (seed + 1000 so they differ from the prefix)."""
    n = w.steps if steps is None else steps
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + 1000)
    dt = torch_dtype(w.dtype)
    q = _randn((n, w.N, w.H, w.d_k), gen, device, 1.0, dt)
    k = _randn((n, w.N, w.H, w.d_k), gen, device, 1.0, dt)
    v = _randn((n, w.N, w.H, w.d_v), gen, device, 1.0, dt)
    return {"q": q, "k": k, "v": v}


def small_integer_inputs(B: int, H: int, T: int, d_k: int, d_v: int, lo: int, hi: int, seed: int,
                         dtype: torch.dtype = torch.bfloat16) -> Dict[str, torch.Tensor]:
    """q, k, v with integer entries drawn uniformly from [lo, hi] (exact in bf16 and fp32)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    out = {}
    for name, d in (("q", d_k), ("k", d_k), ("v", d_v)):
        out[name] = torch.randint(lo, hi + 1, (B, H, T, d), generator=gen).to(dtype)
    return out
