"""GPU parity of lin_attn_decode_step against the fp64 oracle (through the C ABI)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from chunked_causal_linear_k1_amd import binding, inputs, workloads
from chunked_causal_linear_k1_amd.workloads import (PSI_ELU1, PSI_IDENTITY, PSI_PRF, PSI_PRF_QSHIFT, DecodeWorkload,
                                                    Workload)

from gpu_common import announce, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _state_from_prefix(w: DecodeWorkload, prefix, nthreads=0):
    """The oracle's fp64 state after the seeded prefix (keys and values only)."""
    k = prefix["k"].reshape(w.N * w.H, w.prefix_len, w.d_k)
    v = prefix["v"].reshape(w.N * w.H, w.prefix_len, w.d_v)
    gam = [w.gamma] * (w.N * w.H)
    _, S, Z = oracle.prefill(None, k, v, w.psi, gamma=gam, normalize=w.normalize, want_state=True,
                             nthreads=nthreads)
    return S, Z


def _run_steps(w: DecodeWorkload, S, Z, steps, n_steps, prf=None):
    """Run n_steps on the GPU and the oracle from the same fp32 starting state; compare every step."""
    Sg = torch.from_numpy(S.astype(np.float32)).reshape(w.N, w.H, w.n_psi, w.d_v).to(DEV)
    Zg = torch.from_numpy(Z.astype(np.float32)).reshape(w.N, w.H, w.n_psi).to(DEV)
    So = Sg.cpu().double().numpy().reshape(w.N * w.H, w.n_psi, w.d_v).copy()
    Zo = Zg.cpu().double().numpy().reshape(w.N * w.H, w.n_psi).copy()
    gam = [w.gamma] * w.H
    worst = (0.0, 0.0)
    for t in range(n_steps):
        q, k, v = steps["q"][t], steps["k"][t], steps["v"][t]
        o = binding.lin_attn_decode_step(q.to(DEV), k.to(DEV), v.to(DEV), Sg, Zg, psi=w.psi, normalize=w.normalize,
                                         eps=w.eps, gamma=gam, prf_w=None if prf is None else prf.to(DEV))
        ref = oracle.decode_step(q.reshape(-1, w.d_k), k.reshape(-1, w.d_k), v.reshape(-1, w.d_v), So, Zo, w.psi,
                                 prf_w=prf, w_head=None if prf is None else [b % w.H for b in range(w.N * w.H)],
                                 gamma=[w.gamma] * (w.N * w.H), normalize=w.normalize,
                                 eps=float(np.float32(w.eps)))
        rel, mx = assert_close(o.cpu().reshape(-1, w.d_v).numpy(), ref, w.dtype, f"{w.name} step {t}")
        worst = (max(worst[0], rel), max(worst[1], mx))
    torch.cuda.synchronize()
    assert_close(Sg.cpu().reshape(-1, w.n_psi, w.d_v).numpy(), So, w.dtype, f"{w.name} final S")
    if w.normalize:  # without a denominator the normaliser is not maintained
        assert_close(Zg.cpu().reshape(-1, w.n_psi).numpy(), Zo, w.dtype, f"{w.name} final Z")
    return worst


@pytest.mark.parametrize("psi,d,normalize,gamma", [(PSI_ELU1, 128, 1, 0.999), (PSI_IDENTITY, 64, 0, 0.97),
                                                   (PSI_ELU1, 64, 1, 1.0)])
def test_decode_small(psi, d, normalize, gamma):
    w = DecodeWorkload(name=f"dec_psi{psi}_d{d}", N=3, H=5, d_k=d, d_v=d, n_psi=d, psi=psi, normalize=normalize,
                       eps=1e-6, gamma=gamma, prefix_len=200, steps=8, seed=7)
    announce(f"decode small {w.name}")
    prefix = inputs.make_decode_prefix(w)
    S, Z = _state_from_prefix(w, prefix)
    steps = inputs.make_decode_steps(w)
    _run_steps(w, S, Z, steps, w.steps)


@pytest.mark.parametrize("psi,d,normalize,gamma", [(PSI_ELU1, 64, 1, 0.99), (PSI_IDENTITY, 128, 0, 0.97)])
def test_decode_f32(psi, d, normalize, gamma):
    """fp32 inputs (the prefill's fp32 configuration carried into decode): the fp32 bar."""
    w = DecodeWorkload(name=f"dec_f32_psi{psi}_d{d}", N=2, H=3, d_k=d, d_v=d, n_psi=d, psi=psi, normalize=normalize,
                       eps=1e-6, gamma=gamma, prefix_len=100, steps=6, seed=9, dtype="f32")
    announce(f"decode fp32 {w.name}")
    prefix = inputs.make_decode_prefix(w)
    S, Z = _state_from_prefix(w, prefix)
    steps = inputs.make_decode_steps(w)
    _run_steps(w, S, Z, steps, w.steps)


@pytest.mark.parametrize("psi,q_mult", [(PSI_PRF, 1.0), (PSI_PRF_QSHIFT, 1.0), (PSI_PRF_QSHIFT, 8.0)])
def test_decode_prf(psi, q_mult):
    """PRF decode; with the query-row shift also for queries 8x larger, whose unshifted
    log-features (about -300) underflow in fp32."""
    w = DecodeWorkload(name=f"dec_prf{psi}", N=2, H=3, d_k=128, d_v=128, n_psi=256, psi=psi, normalize=1, eps=1e-6,
                       gamma=0.99, prefix_len=64, steps=4, seed=8)
    announce(f"decode prf psi={psi} q x{q_mult}")
    g = torch.Generator().manual_seed(99)
    prf = torch.randn((3, 256, 128), generator=g).to(torch.bfloat16)
    # prefix state from the oracle, with keys scaled like the PRF workload
    pk = (torch.randn((2, 3, 64, 128), generator=g) * 128 ** -0.25).to(torch.bfloat16)
    pv = torch.randn((2, 3, 64, 128), generator=g).to(torch.bfloat16)
    _, S, Z = oracle.prefill(None, pk.reshape(6, 64, 128), pv.reshape(6, 64, 128), PSI_PRF, n_psi=256, prf_w=prf,
                             w_head=[b % 3 for b in range(6)], gamma=[0.99] * 6, normalize=1, want_state=True)
    steps = {n: (torch.randn((4, 2, 3, 128), generator=g) * (128 ** -0.25 if n != "v" else 1.0)).to(torch.bfloat16)
             for n in ("q", "k", "v")}
    steps["q"] = (steps["q"].float() * q_mult).to(torch.bfloat16)  # a power of two: exact
    _run_steps(w, S, Z, steps, 4, prf=prf)


def test_decode_full_size_all_steps():
    """The decode workload as configured: 32 streams x 64 heads, the state of the seeded
    4096-token prefix, all 256 consecutive steps. Every step's output and the final state and
    normaliser against the oracle carried over the same 256 steps."""
    w = workloads.DECODE_32x64
    announce("decode full size: 256 steps from the oracle's prefix state")
    prefix = inputs.make_decode_prefix(w)
    S, Z = _state_from_prefix(w, prefix)
    steps = inputs.make_decode_steps(w)
    assert w.steps == 256 and steps["q"].shape[0] == 256
    rel, mx = _run_steps(w, S, Z, steps, w.steps)
    print(f"[parity] decode_32x64 worst step over 256: rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)


def test_decode_prefix_state_from_prefill():
    """The decode workload's starting state built on the GPU (a prefill of the 4096-token
    prefix with zero queries, final state only), against the oracle's state after the prefix.
    The state has no fixed scale (Z sums about a thousand features), so max-abs is taken after
    scaling by the largest reference magnitude; rel-L2 is unscaled."""
    w = workloads.DECODE_32x64
    announce("decode prefix state from GPU prefill")
    prefix = inputs.make_decode_prefix(w)
    S, Z = _state_from_prefix(w, prefix)
    k, v = prefix["k"].to(DEV), prefix["v"].to(DEV)
    Sg = torch.empty((w.N, w.H, w.n_psi, w.d_v), dtype=torch.float32, device=DEV)
    Zg = torch.empty((w.N, w.H, w.n_psi), dtype=torch.float32, device=DEV)
    binding.lin_attn_prefill(torch.zeros_like(k), k, v, psi=w.psi, chunk=64, normalize=w.normalize, eps=w.eps,
                             gamma=[w.gamma] * w.H, final_S=Sg, final_Z=Zg)
    torch.cuda.synchronize()
    sS, sZ = float(np.abs(S).max()), float(np.abs(Z).max())
    assert_close(Sg.cpu().reshape(-1, w.n_psi, w.d_v).numpy() / sS, S / sS, "bf16",
                 f"prefix state S (scaled by max |S| = {sS:.3g})")
    assert_close(Zg.cpu().reshape(-1, w.n_psi).numpy() / sZ, Z / sZ, "bf16",
                 f"prefix normaliser Z (scaled by max |Z| = {sZ:.3g})")


def test_prefill_to_decode_handoff():
    """GPU prefill's final state, fed to GPU decode, matches the oracle on the whole sequence."""
    P, n, d = 300, 6, 128
    w = Workload(name="handoff", B=2, H=3, T=P + n, d_k=d, d_v=d, n_psi=d, chunk=64, psi=PSI_ELU1, normalize=1,
                 eps=1e-6, dtype="bf16", seed=31, qk_scale=0.5, v_scale=1.0, decay="const:0.999")
    announce("prefill -> decode hand-off")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    gam = list(inp["gamma"])
    qd, kd, vd = (inp[x].to(DEV) for x in ("q", "k", "v"))
    S = torch.empty((2, 3, d, d), dtype=torch.float32, device=DEV)
    Z = torch.empty((2, 3, d), dtype=torch.float32, device=DEV)
    binding.lin_attn_prefill(qd[:, :, :P].contiguous(), kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous(),
                             psi=PSI_ELU1, chunk=64, normalize=1, eps=1e-6, gamma=gam, final_S=S, final_Z=Z)
    outs = []
    for t in range(P, P + n):
        outs.append(binding.lin_attn_decode_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(),
                                                 vd[:, :, t].contiguous(), S, Z, psi=PSI_ELU1, normalize=1,
                                                 eps=1e-6, gamma=gam).cpu())
    got = torch.stack(outs, dim=2).reshape(6, n, d).numpy()
    ref = oracle.prefill(inp["q"].reshape(6, P + n, d), inp["k"].reshape(6, P + n, d), inp["v"].reshape(6, P + n, d),
                         PSI_ELU1, gamma=[gam[b % 3] for b in range(6)], normalize=1, eps=float(np.float32(1e-6)))
    assert_close(got, ref[:, P:], "bf16", "decode after prefill")


@pytest.mark.parametrize("psi,n_psi,gated", [(PSI_ELU1, 128, False), (PSI_IDENTITY, 64, False), (PSI_PRF, 256, False),
                                             (PSI_ELU1, 128, True)])
def test_decode_bf16_output_is_rounded_fp32(psi, n_psi, gated):
    """bf16 outputs of the decode step are the fp32 outputs rounded to nearest even, bit for bit:
    two copies of one state take the same step, one writing fp32 and one bf16, and end in
    bitwise equal states."""
    d = 128 if psi == PSI_PRF else n_psi
    N, H = 4, 6
    announce(f"decode bf16 output psi={psi} n_psi={n_psi} gated={gated}")
    gen = torch.Generator().manual_seed(91 + psi)
    q, k, v = ((torch.randn((N, H, d), generator=gen) * 0.5).to(torch.bfloat16).to(DEV) for _ in range(3))
    S = (torch.randn((N, H, n_psi, d), generator=gen) * 0.1).abs().to(DEV)
    Z = (torch.rand((N, H, n_psi), generator=gen) + 1.0).to(DEV)
    prf = (torch.randn((H, n_psi, d), generator=gen)).to(torch.bfloat16).to(DEV) if psi == PSI_PRF else None
    lg = (torch.rand((N, H, n_psi), generator=gen) * -0.1).to(DEV) if gated else None
    outs, states = [], []
    for dt in (torch.float32, torch.bfloat16):
        S1, Z1 = S.clone(), Z.clone()
        if gated:
            o = binding.lin_attn_decode_step_gated(q, k, v, lg, S1, Z1, psi=psi, normalize=1, prf_w=prf, out_dtype=dt)
        else:
            o = binding.lin_attn_decode_step(q, k, v, S1, Z1, psi=psi, normalize=1, gamma=[0.99] * H, prf_w=prf,
                                             out_dtype=dt)
        torch.cuda.synchronize()
        outs.append(o)
        states.append((S1, Z1))
    assert outs[1].dtype == torch.bfloat16
    assert torch.equal(outs[0].to(torch.bfloat16), outs[1])
    assert torch.equal(states[0][0], states[1][0]) and torch.equal(states[0][1], states[1][1])

