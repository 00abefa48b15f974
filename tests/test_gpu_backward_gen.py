"""GPU parity of the fp32 vector-ALU backward (lin_attn_prefill_backward and its packed form,
through the C ABI) against the fp64 backward oracle (oracle.prefill_backward, the adjoint of the
token loop, pinned on the CPU): the shapes the matrix-core backward does not take, fp32 inputs
(identity, elu+1, random features with and without the query-row shift, d = 64 and 128) and bf16
inputs at d = 64.

Tolerances: fp32 inputs are held to the fp32 forward bar, rel-L2 <= 1e-5 per gradient; bf16 inputs
to the bf16 bar (rel-L2 <= 2e-3, max-abs <= 1e-2 of the largest reference magnitude, as for the
matrix-core backward: gradients have no fixed scale).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from chunked_causal_linear_k1_amd import binding, inputs
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, PSI_PRF, PSI_PRF_QSHIFT, Workload

from gpu_common import BF16_MAX_ABS, BF16_REL_L2, F32_REL_L2, announce, metrics

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(got, ref, dtype, label):
    rel, mx = metrics(got, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs/scale={mx / scale:.3e} scale={scale:.3e}", flush=True)
    if dtype == "f32":
        assert rel <= F32_REL_L2, f"{label}: rel_l2={rel:.3e}"
    else:
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS * scale, f"{label}: rel_l2={rel:.3e} max_abs/scale={mx / scale:.3e}"


def _workload(dtype, psi, n_psi, d, normalize, decay, B, H, T, C, seed):
    if psi in (PSI_PRF, PSI_PRF_QSHIFT):
        scale = d ** -0.25
    elif psi == PSI_IDENTITY:
        scale = d ** -0.5
    else:
        scale = 0.5
    return Workload(name="bwd_gen", B=B, H=H, T=T, d_k=d, d_v=d, n_psi=n_psi, chunk=C, psi=psi, normalize=normalize,
                    eps=1e-6, dtype=dtype, seed=seed, qk_scale=scale, v_scale=1.0, decay=decay)


def _prf(w):
    return w.psi in (PSI_PRF, PSI_PRF_QSHIFT)


def _prefix_state(w, inp, T0, seed):
    """The state after a seeded T0-token prefix (oracle, same bank and decay), as a hand-off gives it."""
    gen = torch.Generator().manual_seed(seed)
    dt = inp["q"].dtype
    BH = w.B * w.H
    k0 = (torch.randn((BH, T0, w.d_k), generator=gen) * w.qk_scale).to(dt)
    v0 = torch.randn((BH, T0, w.d_v), generator=gen).to(dt)
    if w.psi == PSI_IDENTITY and w.normalize:
        k0 = k0.abs()
    g = inp["gamma"]
    kpsi = PSI_PRF if w.psi == PSI_PRF_QSHIFT else w.psi
    _, S, Z = oracle.prefill(None, k0, v0, kpsi, n_psi=w.n_psi, prf_w=inp["prf_w"] if _prf(w) else None,
                             w_head=[b % w.H for b in range(BH)] if _prf(w) else None,
                             gamma=None if g is None else [float(g[b % w.H]) for b in range(BH)],
                             normalize=w.normalize, want_state=True)
    return S.reshape(w.B, w.H, w.n_psi, w.d_v), Z.reshape(w.B, w.H, w.n_psi)


def _oracle(w, q, k, v, dout, inp, S0=None, Z0=None):
    BH = w.B * w.H
    g = inp["gamma"]
    r = lambda x: x.reshape(BH, x.shape[-2], x.shape[-1])  # noqa: E731
    return oracle.prefill_backward(r(q), r(k), r(v), r(dout), w.psi, n_psi=w.n_psi,
                                   prf_w=inp["prf_w"] if _prf(w) else None,
                                   w_head=[b % w.H for b in range(BH)] if _prf(w) else None,
                                   gamma=None if g is None else [float(g[b % w.H]) for b in range(BH)],
                                   normalize=w.normalize, eps=w.eps,
                                   S0=None if S0 is None else S0.reshape(BH, w.n_psi, w.d_v),
                                   Z0=None if Z0 is None else Z0.reshape(BH, w.n_psi))


# name, input dtype, psi, n_psi, d, normalize, decay, B, H, T, C, init state, dout dtype, layout
GEN_CASES = [
    ("f32_retention_d64", "f32", PSI_IDENTITY, 64, 64, 0, "retnet_spread", 1, 4, 300, 64, False, "f32", "bhtd"),
    ("f32_elu1_norm_d64", "f32", PSI_ELU1, 64, 64, 1, "none", 2, 2, 333, 64, False, "f32", "bhtd"),
    ("f32_elu1_norm_decay_state_d128", "f32", PSI_ELU1, 128, 128, 1, "const:0.995", 1, 2, 257, 32, True, "f32",
     "bhtd"),
    ("f32_identity_norm_nonneg_c16", "f32", PSI_IDENTITY, 128, 128, 1, "const:0.98", 1, 2, 100, 16, False, "f32",
     "bhtd"),
    ("f32_prf128_d64", "f32", PSI_PRF, 128, 64, 1, "none", 1, 2, 200, 32, False, "f32", "bhtd"),
    ("f32_qshift128_d64_decay_state", "f32", PSI_PRF_QSHIFT, 128, 64, 1, "const:0.99", 1, 2, 150, 16, True, "f32",
     "bhtd"),
    ("f32_prf64_nonorm_decay", "f32", PSI_PRF, 64, 64, 0, "retnet_spread", 1, 2, 180, 64, False, "f32", "bhtd"),
    ("f32_elu1_bthd_state_d64", "f32", PSI_ELU1, 64, 64, 1, "const:0.99", 2, 3, 210, 64, True, "f32", "bthd"),
    ("f32_retention_many_segments", "f32", PSI_IDENTITY, 64, 64, 0, "const:0.999", 1, 1, 9000, 64, True, "f32",
     "bhtd"),
    # the largest records the query sweep holds in registers (n_psi * d_v = 16384, four blocks per thread)
    ("f32_prf256_d64_decay_state_c16", "f32", PSI_PRF, 256, 64, 1, "const:0.995", 1, 2, 140, 16, True, "f32", "bhtd"),
    ("f32_qshift128_d128_c32", "f32", PSI_PRF_QSHIFT, 128, 128, 1, "none", 1, 1, 120, 32, False, "f32", "bhtd"),
    # widths that are multiples of 4 but not of 16 or 64
    ("f32_elu1_d48", "f32", PSI_ELU1, 48, 48, 1, "const:0.99", 1, 3, 111, 32, True, "f32", "bhtd"),
    ("f32_retention_d20_bthd", "f32", PSI_IDENTITY, 20, 20, 0, "retnet_spread", 2, 2, 77, 16, False, "f32", "bthd"),
    ("bf16_elu1_norm_d64_bf16_dout", "bf16", PSI_ELU1, 64, 64, 1, "none", 2, 2, 300, 64, False, "bf16", "bhtd"),
    ("bf16_retention_d64_c32_state_bthd", "bf16", PSI_IDENTITY, 64, 64, 0, "retnet_spread", 1, 3, 260, 32, True,
     "f32", "bthd"),
    ("bf16_elu1_decay_d64_c128", "bf16", PSI_ELU1, 64, 64, 1, "const:0.995", 1, 2, 400, 128, False, "f32", "bhtd"),
]


@pytest.mark.parametrize("case", GEN_CASES, ids=[c[0] for c in GEN_CASES])
def test_backward_gen_matches_oracle(case):
    name, dt, psi, n_psi, d, normalize, decay, B, H, T, C, with_state, ddt, layout = case
    w = _workload(dt, psi, n_psi, d, normalize, decay, B, H, T, C, seed=500 + [c[0] for c in GEN_CASES].index(name))
    announce(f"backward gen {name} B={B} H={H} T={T} C={C} d={d} n_psi={n_psi} layout={layout}")
    inp = inputs.make_prefill_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    if psi == PSI_IDENTITY and normalize:
        q, k = q.abs(), k.abs()
    dout = inputs.make_upstream_grad((B, H, T, d), w.seed + 11,
                                     dtype=torch.float32 if ddt == "f32" else torch.bfloat16)
    S0 = Z0 = None
    if with_state:
        S0, Z0 = _prefix_state(w, inp, 48, w.seed + 5)
    tr = (lambda x: x.transpose(1, 2).contiguous()) if layout == "bthd" else (lambda x: x.contiguous())
    g = inp["gamma"]
    S0d = None if S0 is None else torch.from_numpy(S0).float().to(DEV)
    Z0d = None if Z0 is None else torch.from_numpy(Z0).float().to(DEV)
    dS0 = torch.zeros((B, H, n_psi, d), device=DEV) if with_state else None
    dZ0 = torch.zeros((B, H, n_psi), device=DEV) if with_state else None
    dq, dk, dv = binding.lin_attn_prefill_backward(
        *(tr(x).to(DEV) for x in (q, k, v, dout)), psi=psi, chunk=C, normalize=normalize, eps=w.eps,
        gamma=None if g is None else list(g), prf_w=inp["prf_w"].to(DEV) if _prf(w) else None, init_S=S0d,
        init_Z=Z0d, dinit_S=dS0, dinit_Z=dZ0, layout=layout)
    torch.cuda.synchronize()
    untr = (lambda x: x.transpose(1, 2)) if layout == "bthd" else (lambda x: x)
    got = [untr(x.cpu()).numpy() for x in (dq, dk, dv)]
    ref = _oracle(w, q, k, v, dout, inp,
                  S0=None if S0d is None else S0d.cpu().double().numpy(),
                  Z0=None if Z0d is None else Z0d.cpu().double().numpy())
    for lab, a, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        _check(a.reshape(r.shape), r, dt, f"{name} {lab}")
    if with_state:
        _check(dS0.cpu().numpy().reshape(ref[3].shape), ref[3], dt, f"{name} dS0")
        if normalize:
            _check(dZ0.cpu().numpy().reshape(ref[4].shape), ref[4], dt, f"{name} dZ0")


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33])
@pytest.mark.parametrize("psi,normalize,decay", [(PSI_ELU1, 1, "const:0.99"), (PSI_IDENTITY, 0, "retnet_spread")])
def test_backward_gen_edge_lengths(T, psi, normalize, decay):
    """fp32 inputs at lengths around one 16-token step of the sweeps (chunk 16: every segment
    boundary is a step boundary). One token with a denominator is the method's degenerate case
    (o_1 = v_1 w / (w + eps)): dq and dk are eps-sized differences of O(1) terms, held to an
    absolute bound at the fp32 rounding level of those terms (1e-6 of dv's scale)."""
    w = _workload("f32", psi, 64, 64, normalize, decay, 1, 2, T, 16, seed=600 + T)
    announce(f"backward gen edge T={T} psi={psi}")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((1, 2, T, 64), w.seed + 1)
    g = inp["gamma"]
    dq, dk, dv = binding.lin_attn_prefill_backward(
        *(inp[x].to(DEV) for x in ("q", "k", "v")), dout.to(DEV), psi=psi, chunk=16, normalize=normalize, eps=w.eps,
        gamma=None if g is None else list(g))
    torch.cuda.synchronize()
    ref = _oracle(w, inp["q"], inp["k"], inp["v"], dout, inp)
    for lab, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        a = a.cpu().numpy().reshape(r.shape)
        if T == 1 and normalize and lab != "dv":
            err = float(np.abs(a - r).max())
            bound = 1e-6 * float(np.abs(ref[2]).max())
            print(f"[parity] gen edge T=1 {lab} max_abs={err:.3e} bound={bound:.3e}", flush=True)
            assert err <= bound, (lab, err, bound)
            continue
        _check(a, r, "f32", f"gen edge T={T} {lab}")


def test_backward_gen_varlen():
    """Packed fp32 sequences of mixed lengths (empty, one token, around a step, several segments) with
    per-sequence initial states: each sequence's gradients against the oracle on that sequence alone;
    an empty sequence's initial-state gradients are zero."""
    lengths = [0, 1, 17, 300, 64, 2049]
    H, N, total = 2, len(lengths), sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    w = _workload("f32", PSI_ELU1, 64, 64, 1, "const:0.995", 1, H, total, 32, seed=650)
    announce(f"backward gen varlen lengths={lengths}")
    inp = inputs.make_prefill_inputs(w)
    packed = [x[0].transpose(0, 1).contiguous() for x in (inp["q"], inp["k"], inp["v"])]  # [total, H, d]
    dout = inputs.make_upstream_grad((total, H, 64), w.seed + 11)
    g = inp["gamma"]
    S0, Z0 = _prefix_state(dataclasses.replace(w, B=N), inp, 40, w.seed + 5)
    S0d, Z0d = torch.from_numpy(S0).float().to(DEV), torch.from_numpy(Z0).float().to(DEV)
    dS0 = torch.full((N, H, 64, 64), float("nan"), device=DEV)
    dZ0 = torch.full((N, H, 64), float("nan"), device=DEV)
    dq, dk, dv = binding.lin_attn_prefill_backward_varlen(
        *(x.to(DEV) for x in packed), dout.to(DEV), torch.from_numpy(cu).to(DEV), max(lengths) + 30, psi=PSI_ELU1,
        chunk=32, normalize=1, eps=w.eps, gamma=list(g), init_S=S0d, init_Z=Z0d, dinit_S=dS0, dinit_Z=dZ0)
    torch.cuda.synchronize()
    got = [x.cpu() for x in (dq, dk, dv)]
    S0r, Z0r = S0d.cpu().double().numpy(), Z0d.cpu().double().numpy()
    for b, L in enumerate(lengths):
        if L == 0:
            assert torch.count_nonzero(dS0[b]).item() == 0 and torch.count_nonzero(dZ0[b]).item() == 0
            continue
        sl = slice(int(cu[b]), int(cu[b + 1]))
        blk = [x[sl].transpose(0, 1).unsqueeze(0) for x in packed + [dout]]  # [1, H, L, d]
        ref = oracle.prefill_backward(*blk[:3], blk[3], PSI_ELU1, gamma=g[None], normalize=1, eps=w.eps,
                                      S0=S0r[b:b + 1], Z0=Z0r[b:b + 1])
        for lab, a, r in zip(("dq", "dk", "dv"), got, ref[:3]):
            _check(a[sl].transpose(0, 1).unsqueeze(0).numpy(), r, "f32", f"gen varlen seq {b} (T={L}) {lab}")
        _check(dS0[b:b + 1].cpu().numpy(), ref[3], "f32", f"gen varlen seq {b} dS0")
        _check(dZ0[b:b + 1].cpu().numpy(), ref[4], "f32", f"gen varlen seq {b} dZ0")


def test_backward_tiny_f32_workload():
    """The tiny fp32 workload's shape (1 x 1 x 1024, d 64, chunk 64, elu+1 with a denominator):
    every gradient against the oracle, and a second call bitwise equal to the first."""
    w = _workload("f32", PSI_ELU1, 64, 64, 1, "none", 1, 1, 1024, 64, seed=0)
    w = dataclasses.replace(w, qk_scale=1.0)
    announce("backward gen tiny f32 workload")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((1, 1, 1024, 64), 17)
    args = [inp[x].to(DEV) for x in ("q", "k", "v")] + [dout.to(DEV)]
    first = binding.lin_attn_prefill_backward(*args, psi=PSI_ELU1, chunk=64, normalize=1, eps=w.eps)
    again = binding.lin_attn_prefill_backward(*args, psi=PSI_ELU1, chunk=64, normalize=1, eps=w.eps)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b), "backward is not deterministic"
    ref = _oracle(w, inp["q"], inp["k"], inp["v"], dout, inp)
    for lab, a, r in zip(("dq", "dk", "dv"), first, ref[:3]):
        _check(a.cpu().numpy().reshape(r.shape), r, "f32", f"tiny f32 {lab}")
