"""GPU parity of the backward pass (lin_attn_prefill_backward, through the C ABI) against the
fp64 backward oracle (oracle.prefill_backward, the adjoint of the token loop, pinned on the CPU).

Cases span both sweeps' paths: identity features with per-head decay and no denominator (the
retention form), elu+1 with and without decay and a denominator, identity with a denominator
(non-negative q and k, so the denominator is a positive sum), chunk 64 and 128, ragged tails,
sequences shorter than one step, many segments (the reverse scan), long segments of many steps,
initial states (and their gradients), bf16 upstream gradients and the [B, T, H, d] layout.

Tolerances: those of the forward pass for bf16 inputs (rel-L2 <= 2e-3), with max-abs applied
after scaling by the largest reference magnitude: gradients have no fixed scale (a query's
gradient grows with the state it reads).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from chunked_causal_linear_k1_amd import binding, inputs, workloads
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, PSI_PRF, PSI_PRF_QSHIFT, Workload

from gpu_common import BF16_MAX_ABS, BF16_REL_L2, announce, metrics

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _check(got, ref, label):
    rel, mx = metrics(got, ref)
    scale = max(float(np.abs(ref).max()), 1e-30)
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs/scale={mx / scale:.3e} scale={scale:.3e}", flush=True)
    assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS * scale, f"{label}: rel_l2={rel:.3e} max_abs/scale={mx / scale:.3e}"


def _workload(psi, normalize, decay, B, H, T, C, seed):
    scale = 128 ** -0.5 if psi == PSI_IDENTITY else 0.5
    return Workload(name="bwd", B=B, H=H, T=T, d_k=128, d_v=128, n_psi=128, chunk=C, psi=psi, normalize=normalize,
                    eps=1e-6, dtype="bf16", seed=seed, qk_scale=scale, v_scale=1.0, decay=decay)


def _prefix_state(w, inp, T0, seed):
    """The state after a seeded T0-token prefix (oracle), as a hand-off would give it."""
    gen = torch.Generator().manual_seed(seed)
    k0 = (torch.randn((w.B, w.H, T0, w.d_k), generator=gen) * w.qk_scale).to(torch.bfloat16)
    v0 = torch.randn((w.B, w.H, T0, w.d_v), generator=gen).to(torch.bfloat16)
    if w.psi == PSI_IDENTITY and w.normalize:
        k0 = k0.abs()
    g = inp["gamma"]
    _, S, Z = oracle.prefill(None, k0, v0, w.psi, gamma=None if g is None else np.repeat(g[None], w.B, 0),
                             normalize=w.normalize, want_state=True)
    return S, Z


# name, psi, normalize, decay, B, H, T, C, init state, dout dtype, layout
CASES = [
    ("retention_decay", PSI_IDENTITY, 0, "retnet_spread", 1, 4, 300, 64, False, "f32", "bhtd"),
    ("retention_c128_state", PSI_IDENTITY, 0, "const:0.99", 1, 2, 1000, 128, True, "f32", "bhtd"),
    ("elu1_norm", PSI_ELU1, 1, "none", 2, 2, 333, 64, False, "f32", "bhtd"),
    ("elu1_norm_decay_state", PSI_ELU1, 1, "const:0.995", 1, 3, 517, 64, True, "f32", "bhtd"),
    ("identity_norm_nonneg", PSI_IDENTITY, 1, "const:0.98", 1, 2, 257, 64, False, "f32", "bhtd"),
    ("elu1_short", PSI_ELU1, 1, "none", 1, 2, 37, 64, False, "f32", "bhtd"),
    ("elu1_bf16_dout_bthd", PSI_ELU1, 1, "const:0.99", 2, 3, 200, 128, True, "bf16", "bthd"),
    ("retention_bthd_bf16", PSI_IDENTITY, 0, "retnet_spread", 1, 4, 450, 64, False, "bf16", "bthd"),
    ("elu1_norm_decay_c32_state", PSI_ELU1, 1, "const:0.99", 1, 2, 333, 32, True, "f32", "bhtd"),
    ("retention_c32_bthd", PSI_IDENTITY, 0, "retnet_spread", 1, 3, 260, 32, False, "bf16", "bthd"),
]


def _run(case):
    name, psi, normalize, decay, B, H, T, C, with_state, dt, layout = case
    w = _workload(psi, normalize, decay, B, H, T, C, seed=100 + [c[0] for c in CASES].index(name))
    announce(f"backward {name} B={B} H={H} T={T} C={C} layout={layout}")
    inp = inputs.make_prefill_inputs(w)
    q, k, v = inp["q"], inp["k"], inp["v"]
    if psi == PSI_IDENTITY and normalize:
        q, k = q.abs(), k.abs()
    ddt = torch.float32 if dt == "f32" else torch.bfloat16
    dout = inputs.make_upstream_grad((B, H, T, 128), w.seed + 11, dtype=ddt)
    g = inp["gamma"]
    gam = None if g is None else list(g)
    S0 = Z0 = None
    if with_state:
        S0, Z0 = _prefix_state(w, inp, 96, w.seed + 5)
    tr = (lambda x: x.transpose(1, 2).contiguous()) if layout == "bthd" else (lambda x: x.contiguous())
    qd, kd, vd, dod = (tr(x).to(DEV) for x in (q, k, v, dout))
    kw = dict(psi=psi, chunk=C, normalize=normalize, eps=w.eps, gamma=gam, layout=layout)
    S0d = None if S0 is None else torch.from_numpy(S0).float().to(DEV)
    Z0d = None if Z0 is None else torch.from_numpy(Z0).float().to(DEV)
    dS0 = torch.zeros((B, H, 128, 128), device=DEV) if with_state else None
    dZ0 = torch.zeros((B, H, 128), device=DEV) if with_state else None
    dq, dk, dv = binding.lin_attn_prefill_backward(qd, kd, vd, dod, init_S=S0d, init_Z=Z0d, dinit_S=dS0,
                                                   dinit_Z=dZ0, **kw)
    torch.cuda.synchronize()
    untr = (lambda x: x.transpose(1, 2)) if layout == "bthd" else (lambda x: x)
    got = [untr(x.cpu()).numpy() for x in (dq, dk, dv)]
    # the oracle takes S0 / Z0 as the same fp32 values the GPU received
    S0r = None if S0 is None else S0d.cpu().double().numpy()
    Z0r = None if Z0 is None else Z0d.cpu().double().numpy()
    ref = oracle.prefill_backward(q, k, v, dout, psi, gamma=None if g is None else np.repeat(g[None], B, 0),
                                  normalize=normalize, eps=w.eps, S0=S0r, Z0=Z0r)
    for lab, a, b in zip(("dq", "dk", "dv"), got, ref[:3]):
        _check(a, b, f"{name} {lab}")
    if with_state:
        _check(dS0.cpu().numpy(), ref[3], f"{name} dS0")
        if normalize:
            _check(dZ0.cpu().numpy(), ref[4], f"{name} dZ0")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    _run(case)


@pytest.mark.parametrize("psi,normalize,decay", [(PSI_IDENTITY, 0, "retnet_spread"), (PSI_ELU1, 1, "const:0.999")])
def test_backward_long_segments(psi, normalize, decay):
    """B*H = 256 sequences of 4100 tokens: segments of 2048 tokens (32 steps each) and a ragged
    third one; sampled heads against the oracle (each head's gradients depend on its own inputs)."""
    B, H, T = 2, 128, 4100
    w = _workload(psi, normalize, decay, B, H, T, 64, seed=21)
    announce(f"backward long segments psi={psi} norm={normalize} B={B} H={H} T={T}")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    dout = inputs.make_upstream_grad((B, H, T, 128), 31, device=DEV)
    g = inp["gamma"]
    kw = dict(psi=psi, chunk=64, normalize=normalize, eps=w.eps, gamma=None if g is None else list(g))
    dq, dk, dv = binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 77), (1, 127)):
        ref = oracle.prefill_backward(inp["q"][b, h].cpu(), inp["k"][b, h].cpu(), inp["v"][b, h].cpu(),
                                      dout[b, h].cpu(), psi, gamma=None if g is None else [g[h]],
                                      normalize=normalize, eps=w.eps)
        for lab, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
            _check(a[b, h].cpu().numpy(), r, f"long b={b} h={h} {lab}")


def test_backward_chunk_invariance():
    """chunks 32, 64 and 128 describe the same function: their gradients agree to rounding."""
    w = _workload(PSI_ELU1, 1, "const:0.99", 1, 2, 700, 64, seed=3)
    announce("backward chunk 64 vs 128 vs 32")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    dout = inputs.make_upstream_grad((1, 2, 700, 128), 4, device=DEV)
    res = []
    for C in (64, 128, 32):
        kw = dict(psi=PSI_ELU1, chunk=C, normalize=1, eps=w.eps, gamma=list(inp["gamma"]))
        res.append(binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw))
    torch.cuda.synchronize()
    for other in (1, 2):
        for lab, a, b in zip(("dq", "dk", "dv"), res[0], res[other]):
            rel, _ = metrics(a.cpu().numpy(), b.cpu().numpy())
            assert rel < 1e-3, (lab, other, rel)


VARLEN_LENGTHS = [200, 0, 1, 63, 64, 65, 777, 128, 1000, 31]
# name, psi, normalize, decay, chunk, dout dtype
VARLEN_CASES = [
    ("elu1_norm_decay", PSI_ELU1, 1, "const:0.995", 64, "f32"),
    ("retention_spread_bf16", PSI_IDENTITY, 0, "retnet_spread", 128, "bf16"),
    ("elu1_norm", PSI_ELU1, 1, "none", 128, "bf16"),
    ("retention_decay_c32", PSI_IDENTITY, 0, "const:0.99", 32, "f32"),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[c[0] for c in VARLEN_CASES])
def test_backward_varlen(case):
    """Packed sequences of mixed lengths (empty, one token, around a step, several segments) with
    per-sequence initial states: each sequence's gradients against the oracle on that sequence alone;
    an empty sequence's initial-state gradients are zero."""
    name, psi, normalize, decay, C, dt = case
    H, N, lengths = 2, len(VARLEN_LENGTHS), VARLEN_LENGTHS
    total = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    w = _workload(psi, normalize, decay, 1, H, total, C, seed=60 + [c[0] for c in VARLEN_CASES].index(name))
    announce(f"backward varlen {name} lengths={lengths} C={C}")
    inp = inputs.make_prefill_inputs(w)  # one [1, H, total, d] stream, cut into sequences below
    packed = [x[0].transpose(0, 1).contiguous() for x in (inp["q"], inp["k"], inp["v"])]  # [total, H, d]
    ddt = torch.float32 if dt == "f32" else torch.bfloat16
    dout = inputs.make_upstream_grad((total, H, 128), w.seed + 11, dtype=ddt)
    g = inp["gamma"]
    wn = dataclasses.replace(w, B=N)
    S0, Z0 = _prefix_state(wn, inp, 96, w.seed + 5)
    S0d = torch.from_numpy(S0).float().to(DEV)
    Z0d = torch.from_numpy(Z0).float().to(DEV)
    dS0 = torch.full((N, H, 128, 128), float("nan"), device=DEV)
    dZ0 = torch.full((N, H, 128), float("nan"), device=DEV)
    dq, dk, dv = binding.lin_attn_prefill_backward_varlen(
        *(x.to(DEV) for x in packed), dout.to(DEV), torch.from_numpy(cu).to(DEV), max(lengths) + 70, psi=psi,
        chunk=C, normalize=normalize, eps=w.eps, gamma=None if g is None else list(g), init_S=S0d, init_Z=Z0d,
        dinit_S=dS0, dinit_Z=dZ0)
    torch.cuda.synchronize()
    got = [x.cpu() for x in (dq, dk, dv)]
    S0r, Z0r = S0d.cpu().double().numpy(), Z0d.cpu().double().numpy()
    for b, L in enumerate(lengths):
        if L == 0:
            assert torch.count_nonzero(dS0[b]).item() == 0
            if normalize:
                assert torch.count_nonzero(dZ0[b]).item() == 0
            continue
        sl = slice(int(cu[b]), int(cu[b + 1]))
        blk = [x[sl].transpose(0, 1).unsqueeze(0) for x in packed + [dout]]  # [1, H, L, d]
        ref = oracle.prefill_backward(*blk[:3], blk[3], psi, gamma=None if g is None else g[None],
                                      normalize=normalize, eps=w.eps, S0=S0r[b:b + 1], Z0=Z0r[b:b + 1])
        for lab, a, r in zip(("dq", "dk", "dv"), got, ref[:3]):
            _check(a[sl].transpose(0, 1).unsqueeze(0).numpy(), r, f"varlen {name} seq {b} (T={L}) {lab}")
        _check(dS0[b:b + 1].cpu().numpy(), ref[3], f"varlen {name} seq {b} dS0")
        if normalize:
            _check(dZ0[b:b + 1].cpu().numpy(), ref[4], f"varlen {name} seq {b} dZ0")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
@pytest.mark.parametrize("psi,normalize,decay", [(PSI_ELU1, 1, "const:0.99"), (PSI_IDENTITY, 0, "retnet_spread")])
def test_backward_edge_lengths(T, psi, normalize, decay):
    """One token, one short of a step, exactly a step, one past it, two steps and one: every
    gradient against the oracle.

    One token with a denominator is the method's degenerate case: o_1 = v_1 w / (w + eps) with
    w = psi(q_1) . psi(k_1), so o_1 depends on q_1 and k_1 only through eps, and dq, dk are
    eps-sized differences of O(1) terms (about 1e-9 here). There they are held to an absolute
    bound at the rounding level of those terms (1e-5 of dv's scale) instead of a relative one."""
    w = _workload(psi, normalize, decay, 1, 2, T, 64, seed=70 + T)
    announce(f"backward edge T={T} psi={psi}")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((1, 2, T, 128), w.seed + 1)
    g = inp["gamma"]
    dq, dk, dv = binding.lin_attn_prefill_backward(
        *(inp[x].to(DEV) for x in ("q", "k", "v")), dout.to(DEV), psi=psi, chunk=64, normalize=normalize, eps=w.eps,
        gamma=None if g is None else list(g))
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], dout, psi,
                                  gamma=None if g is None else np.repeat(g[None], 1, 0), normalize=normalize, eps=w.eps)
    for lab, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        if T == 1 and normalize and lab != "dv":
            err = float(np.abs(a.cpu().numpy() - r).max())
            bound = 1e-5 * float(np.abs(ref[2]).max())
            print(f"[parity] edge T=1 {lab} max_abs={err:.3e} bound={bound:.3e}", flush=True)
            assert err <= bound, (lab, err, bound)
            continue
        _check(a.cpu().numpy(), r, f"edge T={T} {lab}")


def _full_backward(w, heads):
    """The timed backward workload at full size: sampled heads against the oracle, and a second
    call bitwise equal to the first (the backward is deterministic)."""
    announce(f"backward full-size {w.name} sampled heads {heads}")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    dout = inputs.make_upstream_grad((w.B, w.H, w.T, w.d_v), w.seed + 17, device=DEV)
    g = inp["gamma"]
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g))
    first = binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    again = binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b), "backward is not deterministic"
    del again
    for hflat in heads:
        b, h = divmod(hflat, w.H)
        ref = oracle.prefill_backward(inp["q"][b, h].cpu(), inp["k"][b, h].cpu(), inp["v"][b, h].cpu(),
                                      dout[b, h].cpu(), w.psi, gamma=None if g is None else [g[h]],
                                      normalize=w.normalize, eps=w.eps)
        for lab, a, r in zip(("dq", "dk", "dv"), first, ref[:3]):
            _check(a[b, h].cpu().numpy(), r, f"{w.name} b={b} h={h} {lab}")


def test_full_backward_retnet_128k_sampled():
    # the fastest-decaying head and the slowest
    _full_backward(workloads.RETNET_128K, heads=[0, 63])


def test_full_backward_8k_elu1_sampled():
    _full_backward(workloads.PREFILL_8K, heads=[0, 37])


def test_backward_max_decay_heads():
    """256 heads, each with its own decay: every head's gradients against the oracle."""
    w = _workload(PSI_IDENTITY, 0, "retnet_spread", 1, 256, 100, 64, seed=43)
    announce("backward 256 decayed heads")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((1, 256, 100, 128), 44)
    g = inp["gamma"]
    dq, dk, dv = binding.lin_attn_prefill_backward(*(inp[x].to(DEV) for x in ("q", "k", "v")), dout.to(DEV),
                                                   psi=PSI_IDENTITY, chunk=64, normalize=0, eps=w.eps, gamma=list(g))
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(inp["q"], inp["k"], inp["v"], dout, PSI_IDENTITY, gamma=np.asarray(g)[None],
                                  normalize=0, eps=w.eps)
    for lab, a, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3]):
        _check(a.cpu().numpy(), r, f"256 heads {lab}")


# ---- positive random features (psi(x)_p = exp(w_p . x - |x|^2/2) / sqrt(n_psi), one bf16 bank per
# head), with and without the query-row shift: the feature Jacobians on top of the sweeps

def _prf_workload(psi, n_psi, normalize, decay, B, H, T, C, seed):
    return Workload(name="bwd_prf", B=B, H=H, T=T, d_k=128, d_v=128, n_psi=n_psi, chunk=C, psi=psi,
                    normalize=normalize, eps=1e-6, dtype="bf16", seed=seed, qk_scale=128 ** -0.25, v_scale=1.0,
                    decay=decay)


def _prf_backward(w, inp, dout, S0=None, Z0=None, layout="bhtd", q_mult=1.0, label=""):
    """GPU backward (through the C ABI) against the oracle's; returns nothing, asserts the bar."""
    B, H, T = w.B, w.H, w.T
    q = inp["q"] if q_mult == 1.0 else (inp["q"].float() * q_mult).to(torch.bfloat16)  # a power of two: exact
    k, v, W = inp["k"], inp["v"], inp["prf_w"]
    g = inp["gamma"]
    tr = (lambda x: x.transpose(1, 2).contiguous()) if layout == "bthd" else (lambda x: x.contiguous())
    qd, kd, vd, dod = (tr(x).to(DEV) for x in (q, k, v, dout))
    with_state = S0 is not None
    S0d = None if S0 is None else torch.from_numpy(np.ascontiguousarray(S0)).float().to(DEV)
    Z0d = None if Z0 is None else torch.from_numpy(np.ascontiguousarray(Z0)).float().to(DEV)
    dS0 = torch.zeros((B, H, w.n_psi, 128), device=DEV) if with_state else None
    dZ0 = torch.zeros((B, H, w.n_psi), device=DEV) if with_state else None
    dq, dk, dv = binding.lin_attn_prefill_backward(qd, kd, vd, dod, psi=w.psi, chunk=w.chunk, normalize=w.normalize,
                                                   eps=w.eps, gamma=None if g is None else list(g), prf_w=W.to(DEV),
                                                   init_S=S0d, init_Z=Z0d, dinit_S=dS0, dinit_Z=dZ0, layout=layout)
    torch.cuda.synchronize()
    untr = (lambda x: x.transpose(1, 2)) if layout == "bthd" else (lambda x: x)
    got = [untr(x.cpu()).reshape(B * H, T, 128).numpy() for x in (dq, dk, dv)]
    BH = B * H
    ref = oracle.prefill_backward(q.reshape(BH, T, 128), k.reshape(BH, T, 128), v.reshape(BH, T, 128),
                                  dout.reshape(BH, T, 128), w.psi, n_psi=w.n_psi, prf_w=W,
                                  w_head=[b % H for b in range(BH)],
                                  gamma=None if g is None else [float(g[b % H]) for b in range(BH)],
                                  normalize=w.normalize, eps=w.eps,
                                  S0=None if S0d is None else S0d.cpu().double().numpy().reshape(BH, w.n_psi, 128),
                                  Z0=None if Z0d is None else Z0d.cpu().double().numpy().reshape(BH, w.n_psi))
    for lab, a, r in zip(("dq", "dk", "dv"), got, ref[:3]):
        _check(a, r, f"{label} {lab}")
    if with_state:
        _check(dS0.cpu().numpy().reshape(BH, w.n_psi, 128), ref[3], f"{label} dS0")
        if w.normalize:
            _check(dZ0.cpu().numpy().reshape(BH, w.n_psi), ref[4], f"{label} dZ0")


def _prf_state(w, inp, T0, seed):
    """The state after a seeded T0-token prefix with the same bank (oracle), as a hand-off gives it."""
    gen = torch.Generator().manual_seed(seed)
    k0 = (torch.randn((w.B * w.H, T0, 128), generator=gen) * w.qk_scale).to(torch.bfloat16)
    v0 = torch.randn((w.B * w.H, T0, 128), generator=gen).to(torch.bfloat16)
    g = inp["gamma"]
    _, S, Z = oracle.prefill(None, k0, v0, PSI_PRF, n_psi=w.n_psi, prf_w=inp["prf_w"],
                             w_head=[b % w.H for b in range(w.B * w.H)],
                             gamma=None if g is None else [float(g[b % w.H]) for b in range(w.B * w.H)],
                             normalize=w.normalize, want_state=True)
    return S.reshape(w.B, w.H, w.n_psi, 128), Z.reshape(w.B, w.H, w.n_psi)


# name, psi, n_psi, normalize, decay, B, H, T, C, init state, dout dtype, layout, query multiplier
PRF_CASES = [
    ("prf256_norm", PSI_PRF, 256, 1, "none", 1, 2, 300, 64, False, "f32", "bhtd", 1.0),
    ("prf128_norm_decay", PSI_PRF, 128, 1, "const:0.99", 2, 1, 333, 64, False, "f32", "bhtd", 1.0),
    ("prf256_nonorm_decay", PSI_PRF, 256, 0, "retnet_spread", 1, 3, 200, 128, False, "f32", "bhtd", 1.0),
    ("prf256_state_c32", PSI_PRF, 256, 1, "const:0.995", 1, 2, 257, 32, True, "f32", "bhtd", 1.0),
    ("prf128_bf16_dout_bthd", PSI_PRF, 128, 1, "const:0.98", 2, 2, 190, 128, True, "bf16", "bthd", 1.0),
    ("qshift256", PSI_PRF_QSHIFT, 256, 1, "none", 1, 2, 300, 64, False, "f32", "bhtd", 1.0),
    ("qshift128_decay_state", PSI_PRF_QSHIFT, 128, 1, "const:0.99", 1, 2, 222, 64, True, "f32", "bhtd", 1.0),
    # queries 4x larger: the shift keeps every query feature finite (the largest is 1/sqrt(n_psi))
    ("qshift256_large_queries", PSI_PRF_QSHIFT, 256, 1, "const:0.995", 1, 2, 200, 64, False, "f32", "bhtd", 4.0),
    # 141 steps of 64 tokens: the per-step records take the many-segment scan, forward and reversed
    ("prf128_many_steps_state", PSI_PRF, 128, 1, "const:0.999", 1, 1, 9000, 64, True, "f32", "bhtd", 1.0),
]


@pytest.mark.parametrize("case", PRF_CASES, ids=[c[0] for c in PRF_CASES])
def test_backward_prf(case):
    name, psi, n_psi, normalize, decay, B, H, T, C, with_state, dt, layout, q_mult = case
    w = _prf_workload(psi, n_psi, normalize, decay, B, H, T, C, seed=300 + [c[0] for c in PRF_CASES].index(name))
    announce(f"backward prf {name} B={B} H={H} T={T} C={C} n_psi={n_psi} layout={layout}")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((B, H, T, 128), w.seed + 11,
                                     dtype=torch.float32 if dt == "f32" else torch.bfloat16)
    S0 = Z0 = None
    if with_state:
        S0, Z0 = _prf_state(w, inp, 80, w.seed + 5)
    _prf_backward(w, inp, dout, S0=S0, Z0=Z0, layout=layout, q_mult=q_mult, label=name)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_backward_prf_edge_lengths(T):
    """Random features at lengths around one 64-token step (one token: the degenerate case of a
    denominator, its dq and dk are eps-sized; held like the other feature maps' edge cases)."""
    w = _prf_workload(PSI_PRF, 256, 1, "const:0.99", 1, 2, T, 64, seed=400 + T)
    announce(f"backward prf edge T={T}")
    inp = inputs.make_prefill_inputs(w)
    dout = inputs.make_upstream_grad((1, 2, T, 128), w.seed + 11)
    if T == 1:  # o_1 = v_1 w / (w + eps): dq and dk are eps-sized differences, held to an absolute bound
        dq, dk, dv = binding.lin_attn_prefill_backward(*(inp[x].to(DEV) for x in ("q", "k", "v")), dout.to(DEV),
                                                       psi=PSI_PRF, chunk=64, normalize=1, eps=w.eps,
                                                       gamma=list(inp["gamma"]), prf_w=inp["prf_w"].to(DEV))
        torch.cuda.synchronize()
        ref = oracle.prefill_backward(inp["q"].reshape(2, 1, 128), inp["k"].reshape(2, 1, 128),
                                      inp["v"].reshape(2, 1, 128), dout.reshape(2, 1, 128), PSI_PRF, n_psi=256,
                                      prf_w=inp["prf_w"], w_head=[0, 1], gamma=[float(x) for x in inp["gamma"]],
                                      normalize=1, eps=w.eps)
        _check(dv.cpu().reshape(2, 1, 128).numpy(), ref[2], "prf edge T=1 dv")
        # dq and dk are the difference of two terms that cancel to an eps-sized result; the
        # bound is the rounding level (two-term bf16 operands, about 2^-16) of either term:
        # (dout . v / den) sum_p psi(q)_p psi(k)_p (w_p - x), x = q or k
        W = inp["prf_w"].double().numpy()
        for lab, a, r in (("dq", dq, ref[0]), ("dk", dk, ref[1])):
            err = float(np.abs(a.cpu().reshape(2, 1, 128).numpy() - r).max())
            mag = 0.0
            for h in range(2):
                qh, kh = (inp[x][0, h, 0].double().numpy() for x in ("q", "k"))
                g = oracle.feature(qh, PSI_PRF, 256, W[h])
                f = oracle.feature(kh, PSI_PRF, 256, W[h])
                den = float(g @ f) + float(np.float32(w.eps))
                t1 = float(dout[0, h, 0].double().numpy() @ inp["v"][0, h, 0].double().numpy()) / den
                x = qh if lab == "dq" else kh
                mag = max(mag, float(np.abs(t1 * ((g * f) @ W[h] - (g @ f) * x)).max()))
            print(f"[parity] prf edge T=1 {lab} max_abs={err:.3e} (bound {3e-5 * mag:.3e}, term {mag:.3e})",
                  flush=True)
            assert err <= 3e-5 * mag, (lab, err, mag)
        return
    _prf_backward(w, inp, dout, label=f"prf edge T={T}")


def test_full_backward_prf_4k_sampled():
    """The 4k random-feature workload (8 x 16 heads, n_psi 256) at full size: sampled heads against
    the oracle, and a second call bitwise equal to the first."""
    w = workloads.PRF_4K
    heads = [0, 77]
    announce(f"backward full-size {w.name} sampled heads {heads}")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    dout = inputs.make_upstream_grad((w.B, w.H, w.T, w.d_v), w.seed + 17, device=DEV)
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, prf_w=inp["prf_w"])
    first = binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    again = binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b), "backward is not deterministic"
    del again
    W = inp["prf_w"].cpu()
    for hflat in heads:
        b, h = divmod(hflat, w.H)
        ref = oracle.prefill_backward(inp["q"][b, h].cpu(), inp["k"][b, h].cpu(), inp["v"][b, h].cpu(),
                                      dout[b, h].cpu(), w.psi, n_psi=w.n_psi, prf_w=W, w_head=[h],
                                      normalize=w.normalize, eps=w.eps)
        for lab, a, r in zip(("dq", "dk", "dv"), first, ref[:3]):
            _check(a[b, h].cpu().numpy(), r, f"{w.name} b={b} h={h} {lab}")
