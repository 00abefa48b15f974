"""Named synthetic workloads for chunkwise causal linear attention.

Each workload fixes the shapes, the feature map, the decay, the normalisation and
the input distribution. The shapes follow the pages' long-context settings:
"Log-Depth Chunked Linear-Attention Scan" (Implementation notes: chunk sizes 32/64,
sequence lengths 2K..131K), "Linear Attention and Retentive Networks" (Multi-Scale
Decay Formulation: per-head gamma = 1 - 2^(-5-h)), and "Linearized 2-Simplicial
Attention" (section 3.2: positive random features). Nothing here computes any part
of the method; it only names sizes and distributions.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

PSI_IDENTITY = 0
PSI_ELU1 = 1
PSI_PRF = 2
PSI_PRF_QSHIFT = 3  # positive random features with the query-row log-space shift

PSI_NAMES = {PSI_IDENTITY: "identity", PSI_ELU1: "elu+1", PSI_PRF: "prf", PSI_PRF_QSHIFT: "prf+qshift"}


@dataclass(frozen=True)
class Workload:
    """One prefill workload: q, k, v are [B, H, T, d] contiguous."""

    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    n_psi: int
    chunk: int
    psi: int
    normalize: int
    eps: float
    dtype: str  # "bf16" or "f32": storage type of q, k, v (and the PRF bank)
    seed: int
    qk_scale: float  # q, k = N(0,1) * qk_scale
    v_scale: float  # v = N(0,1) * v_scale
    decay: str = "none"  # "none" | "retnet_spread" (gamma_h = 1 - 2^(-5 - 5h/(H-1))) | "const:<g>"
    extra: dict = field(default_factory=dict)

    @property
    def n_chunks(self) -> int:
        return -(-self.T // self.chunk)

    @property
    def token_heads(self) -> int:
        return self.B * self.H * self.T

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


@dataclass(frozen=True)
class DecodeWorkload:
    """Batched single-token decode: N streams x H heads, fp32 state carried in place."""

    name: str
    N: int
    H: int
    d_k: int
    d_v: int
    n_psi: int
    psi: int
    normalize: int
    eps: float
    gamma: float
    prefix_len: int
    steps: int
    seed: int
    dtype: str = "bf16"


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of N sequences of seeded lengths (a serving prefill): q, k, v are
    [total, H, d] with sequence b at tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1. Lengths are
    drawn uniformly from [len_min, len_max] (inputs.varlen_lengths)."""

    name: str
    N: int
    H: int
    len_min: int
    len_max: int
    d_k: int
    d_v: int
    n_psi: int
    chunk: int
    psi: int
    normalize: int
    eps: float
    dtype: str
    seed: int
    qk_scale: float
    v_scale: float
    decay: str = "none"


# Tiny fp32 case the oracle finishes in well under a second.
TINY_F32 = Workload(
    name="tiny_f32_elu1", B=1, H=1, T=1024, d_k=64, d_v=64, n_psi=64, chunk=64,
    psi=PSI_ELU1, normalize=1, eps=1e-6, dtype="f32", seed=0, qk_scale=1.0, v_scale=1.0)

# Training/prefill shape, elu+1, no decay.
PREFILL_8K = Workload(
    name="prefill_8k_elu1", B=4, H=16, T=8192, d_k=128, d_v=128, n_psi=128, chunk=64,
    psi=PSI_ELU1, normalize=1, eps=1e-6, dtype="bf16", seed=1, qk_scale=0.5, v_scale=0.5)

# Positive random features, n_psi = 256 != d_v.
PRF_4K = Workload(
    name="prf256_4k", B=8, H=16, T=4096, d_k=128, d_v=128, n_psi=256, chunk=64,
    psi=PSI_PRF, normalize=1, eps=1e-6, dtype="bf16", seed=2, qk_scale=128 ** -0.25, v_scale=1.0)

# RetNet-style decayed retention at 128k, ragged T (131035 = 1023*128 + 91), no denominator.
RETNET_128K = Workload(
    name="retnet_128k_ragged", B=1, H=64, T=131035, d_k=128, d_v=128, n_psi=128, chunk=128,
    psi=PSI_IDENTITY, normalize=0, eps=1e-6, dtype="bf16", seed=3, qk_scale=128 ** -0.5, v_scale=1.0,
    decay="retnet_spread")

# Serving decode: 32 streams x 64 heads, state pre-filled from a 4096-token prefix.
DECODE_32x64 = DecodeWorkload(
    name="decode_32x64", N=32, H=64, d_k=128, d_v=128, n_psi=128, psi=PSI_ELU1, normalize=1,
    eps=1e-6, gamma=0.999, prefix_len=4096, steps=256, seed=4)

# Data-dependent forget gates (gated linear attention), 8k tokens: one gate per token and key
# feature, log alpha = logsigmoid(z) / 16 with z ~ N(0, 1) (inputs.make_log_gates), no
# denominator, chunks of 16 on the fp32 path.
GATED_8K = Workload(
    name="gated_8k", B=4, H=16, T=8192, d_k=128, d_v=128, n_psi=128, chunk=32, psi=PSI_IDENTITY, normalize=0,
    eps=1e-6, dtype="bf16", seed=7, qk_scale=128 ** -0.5, v_scale=1.0, extra={"gate_temp": 16.0})

# Serving prefill: 32 prompts of 1k..16k tokens packed in one call, retention form as above.
VARLEN_32 = VarlenWorkload(
    name="varlen_32x1k_16k_retention", N=32, H=32, len_min=1024, len_max=16384, d_k=128, d_v=128, n_psi=128,
    chunk=128, psi=PSI_IDENTITY, normalize=0, eps=1e-6, dtype="bf16", seed=5, qk_scale=128 ** -0.5, v_scale=1.0,
    decay="retnet_spread")

PREFILL_WORKLOADS = {w.name: w for w in (TINY_F32, PREFILL_8K, PRF_4K, RETNET_128K)}
