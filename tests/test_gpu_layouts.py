"""GPU parity of the prefill's input/output variants (through the C ABI):

- the [B, T, H, d] token layout: bitwise equal to the [B, H, T, d] call on the same data
  (same kernels, same decomposition, only the addressing differs) and within tolerance of
  the fp64 oracle;
- bf16 output: bitwise equal to the fp32 output rounded to nearest even;
- packed variable-length batches (cu_seqlens): every sequence against the oracle run on
  that sequence alone, with per-sequence initial and final states, including empty
  sequences, sequences shorter than a chunk, exact multiples of the chunk and ragged
  tails;
- the serving hand-off: decode steps continuing from the final states of a packed
  prefill match the oracle run over prefix + new tokens.
Every kernel family is covered: the eight-wave output kernel (C 64, d 128), the
shared-score kernel (C 128 identity), the per-wave-score kernel (C 128 elu+1), d 64,
positive random features and the fp32 path.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from chunked_causal_linear_k1_amd import binding, inputs
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, PSI_PRF, Workload

from gpu_common import announce, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# name, d, n_psi, C, psi, normalize, decay, dtype
CASES = [
    ("elu1_c64_d128", 128, 128, 64, PSI_ELU1, 1, "const:0.995", "bf16"),
    ("retention_c128_d128", 128, 128, 128, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    ("elu1_c128_d128", 128, 128, 128, PSI_ELU1, 1, "none", "bf16"),
    ("identity_c64_d64", 64, 64, 64, PSI_IDENTITY, 0, "const:0.97", "bf16"),
    ("prf256_c64", 128, 256, 64, PSI_PRF, 1, "none", "bf16"),
    # chunks of 32 and PRF at 128: the same 64-token steps, segments on multiples of 64 tokens
    ("retention_c32_d128", 128, 128, 32, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    ("prf256_c128", 128, 256, 128, PSI_PRF, 1, "none", "bf16"),
    ("f32_elu1_c32_d64", 64, 64, 32, PSI_ELU1, 1, "const:0.99", "f32"),
]


def _workload(case, B, H, T, seed):
    name, d, n_psi, C, psi, normalize, decay, dt = case
    scale = d ** -0.5 if psi == PSI_IDENTITY else ((1.0 / d) ** 0.25 if psi == PSI_PRF else 0.5)
    return Workload(name=name, B=B, H=H, T=T, d_k=d, d_v=d, n_psi=n_psi, chunk=C, psi=psi, normalize=normalize,
                    eps=1e-6, dtype=dt, seed=seed, qk_scale=scale, v_scale=1.0, decay=decay)


def _call(w, q, k, v, inp, **kw):
    g = inp["gamma"]
    prf = inp["prf_w"]
    o = binding.lin_attn_prefill(q, k, v, psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps,
                                 gamma=None if g is None else list(g), prf_w=None if prf is None else prf.to(DEV),
                                 **kw)
    torch.cuda.synchronize()
    return o


def _oracle_blocks(w, q, k, v, inp, heads, S0=None, Z0=None, want_state=False):
    """Oracle over blocks q, k, v [nblk, T, d] (CPU tensors); heads[i] is block i's head index."""
    g = inp["gamma"]
    prf = inp["prf_w"]
    return oracle.prefill(q, k, v, w.psi, n_psi=w.n_psi, prf_w=None if prf is None else prf.cpu(),
                          w_head=heads if prf is not None else None,
                          gamma=None if g is None else [float(g[h]) for h in heads], normalize=w.normalize,
                          eps=float(np.float32(w.eps)), S0=S0, Z0=Z0, want_state=want_state)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bthd_layout(case):
    B, H, T = 2, 3, 333
    w = _workload(case, B, H, T, seed=21)
    announce(f"layout bthd {w.name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    n_psi = w.n_psi
    fS1 = torch.empty((B, H, n_psi, w.d_v), dtype=torch.float32, device=DEV)
    fZ1 = torch.empty((B, H, n_psi), dtype=torch.float32, device=DEV)
    fS2, fZ2 = torch.empty_like(fS1), torch.empty_like(fZ1)
    o1 = _call(w, q, k, v, inp, final_S=fS1, final_Z=fZ1)
    qt, kt, vt = (x.transpose(1, 2).contiguous() for x in (q, k, v))
    o2 = _call(w, qt, kt, vt, inp, final_S=fS2, final_Z=fZ2, layout="bthd")
    assert o2.shape == (B, T, H, w.d_v)
    assert torch.equal(o2.transpose(1, 2), o1), "[B,T,H,d] and [B,H,T,d] calls differ"
    assert torch.equal(fS1, fS2)
    if w.normalize:
        assert torch.equal(fZ1, fZ2)
    ref = _oracle_blocks(w, inp["q"].reshape(B * H, T, -1), inp["k"].reshape(B * H, T, -1),
                         inp["v"].reshape(B * H, T, -1), inp, [b % H for b in range(B * H)])
    got = o2.transpose(1, 2).cpu().reshape(B * H, T, w.d_v).numpy()
    if w.psi == PSI_PRF and not w.normalize:
        got, ref = got / np.abs(ref).max(), ref / np.abs(ref).max()
    assert_close(got, ref, w.dtype, f"bthd {w.name}")


@pytest.mark.parametrize("case", [c for c in CASES if c[7] == "bf16"], ids=[c[0] for c in CASES if c[7] == "bf16"])
@pytest.mark.parametrize("layout", ["bhtd", "bthd"])
def test_bf16_output_is_rounded_fp32(case, layout):
    B, H, T = 1, 2, 517
    w = _workload(case, B, H, T, seed=22)
    announce(f"bf16 output {w.name} {layout}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    q, k, v = (inp[x].to(DEV) for x in ("q", "k", "v"))
    if layout == "bthd":
        q, k, v = (x.transpose(1, 2).contiguous() for x in (q, k, v))
    o32 = _call(w, q, k, v, inp, layout=layout)
    o16 = _call(w, q, k, v, inp, layout=layout, out_dtype=torch.bfloat16)
    assert o16.dtype == torch.bfloat16 and o16.shape == o32.shape
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 output is not the fp32 output rounded to nearest even"


def _packed(w, lengths, seed):
    """Packed [total, H, d] inputs: sequence b is an independent seeded draw of lengths[b] tokens."""
    H = w.H
    qs, ks, vs = [], [], []
    prf = gamma = None
    for b, L in enumerate(lengths):
        wb = dataclasses.replace(w, B=1, T=max(L, 1), seed=seed + 97 * b)
        ib = inputs.make_prefill_inputs(wb, device="cpu")
        for lst, key in ((qs, "q"), (ks, "k"), (vs, "v")):
            lst.append(ib[key][0, :, :L].transpose(0, 1))  # [L, H, d]
        if b == 0:
            prf, gamma = ib["prf_w"], ib["gamma"]
    cat = lambda xs: torch.cat(xs, 0).contiguous()
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return {"q": cat(qs), "k": cat(ks), "v": cat(vs), "prf_w": prf, "gamma": gamma}, cu


def _seq(x, cu, b):
    """Sequence b of a packed [total, H, d] tensor as oracle blocks [H, L, d]."""
    return x[int(cu[b]):int(cu[b + 1])].transpose(0, 1).contiguous()


VARLEN_LENGTHS = [200, 0, 1, 63, 64, 65, 777, 128, 1000, 31]


def _prefix_states(w, inp, N, H, seed, P=256):
    """Initial states as a hand-off carries them: the oracle's (fp32-rounded) state after a seeded
    P-token prefix per (sequence, head), same feature map, bank and decay.

    An arbitrary fp32 state with random signs is not used: for a sequence of a few tokens the
    output is then psi(q) . S0, a sum whose terms have unrelated signs, and its relative error is
    that of the single bf16 rounding of psi(q) itself (about 2e-3 rms for elu+1), at the bf16
    tolerance. States built from tokens make these sums coherent, as in every real hand-off."""
    wp = dataclasses.replace(w, B=N, T=P, seed=seed)
    ip = inputs.make_prefill_inputs(wp, device="cpu")
    heads = [b % H for b in range(N * H)]
    _, S, Z = _oracle_blocks(dataclasses.replace(w, normalize=1), None, ip["k"].reshape(N * H, P, -1),
                             ip["v"].reshape(N * H, P, -1), inp, heads, want_state=True)
    return (S.astype(np.float32).reshape(N, H, w.n_psi, w.d_v), Z.astype(np.float32).reshape(N, H, w.n_psi))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_varlen_packed(case):
    H = 2
    lengths = VARLEN_LENGTHS
    N = len(lengths)
    w = _workload(case, N, H, max(lengths), seed=23)
    announce(f"varlen {w.name} lengths={lengths}")
    inp, cu = _packed(w, lengths, seed=300)
    n_psi, d_v = w.n_psi, w.d_v
    S0, Z0 = _prefix_states(w, inp, N, H, seed=400)
    fS = torch.full((N, H, n_psi, d_v), float("nan"), dtype=torch.float32, device=DEV)
    fZ = torch.full((N, H, n_psi), float("nan"), dtype=torch.float32, device=DEV)
    cu_d = torch.from_numpy(cu).to(DEV)
    g = inp["gamma"]
    # a max_seqlen above the longest sequence only adds empty segments
    o = binding.lin_attn_prefill_varlen(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), cu_d,
                                        max(lengths) + 100, psi=w.psi, chunk=w.chunk, normalize=w.normalize,
                                        eps=w.eps, gamma=None if g is None else list(g),
                                        prf_w=None if inp["prf_w"] is None else inp["prf_w"].to(DEV),
                                        init_S=torch.from_numpy(S0).to(DEV), init_Z=torch.from_numpy(Z0).to(DEV),
                                        final_S=fS, final_Z=fZ)
    torch.cuda.synchronize()
    oc = o.cpu()
    for b, L in enumerate(lengths):
        if L == 0:  # no tokens: the final state is the initial state, exactly
            assert torch.equal(fS[b].cpu(), torch.from_numpy(S0[b]))
            if w.normalize:
                assert torch.equal(fZ[b].cpu(), torch.from_numpy(Z0[b]))
            continue
        ref, rS, rZ = _oracle_blocks(w, _seq(inp["q"], cu, b), _seq(inp["k"], cu, b), _seq(inp["v"], cu, b), inp,
                                     list(range(H)), S0=S0[b].astype(np.float64), Z0=Z0[b].astype(np.float64),
                                     want_state=True)
        got = _seq(oc, cu, b).numpy()
        gS, gZ = fS[b].cpu().numpy(), fZ[b].cpu().numpy()
        if w.psi == PSI_PRF:  # no fixed output scale for the state: compare relative to its largest entry
            sc = np.abs(rS).max()
            gS, rS = gS / sc, rS / sc
            zc = np.abs(rZ).max()
            gZ, rZ = gZ / zc, rZ / zc
        assert_close(got, ref, w.dtype, f"varlen {w.name} seq {b} (T={L})")
        assert_close(gS, rS, w.dtype, f"varlen {w.name} seq {b} final S")
        if w.normalize:
            assert_close(gZ, rZ, w.dtype, f"varlen {w.name} seq {b} final Z")


@pytest.mark.parametrize("psi,d,normalize,decay", [(PSI_ELU1, 128, 1, "const:0.999"), (PSI_IDENTITY, 64, 0, "none")])
def test_varlen_prefill_then_decode(psi, d, normalize, decay):
    """Serving hand-off: prefill a packed batch of prompts, then decode new tokens per sequence
    from the prefill's final states; every decode output matches the oracle over the whole
    sequence (prompt + generated tokens)."""
    H, C = 3, 64
    lengths = [130, 5, 64, 300]
    N = len(lengths)
    case = ("handoff", d, d, C, psi, normalize, decay, "bf16")
    w = _workload(case, N, H, max(lengths), seed=24)
    announce(f"varlen prefill -> decode psi={psi} d={d}")
    inp, cu = _packed(w, lengths, seed=500)
    g = inp["gamma"]
    gam = None if g is None else list(g)
    S = torch.empty((N, H, d, d), dtype=torch.float32, device=DEV)
    Z = torch.empty((N, H, d), dtype=torch.float32, device=DEV)
    binding.lin_attn_prefill_varlen(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV),
                                    torch.from_numpy(cu).to(DEV), max(lengths), psi=psi, chunk=C,
                                    normalize=normalize, eps=w.eps, gamma=gam, final_S=S, final_Z=Z)
    steps = 4
    gen = torch.Generator().manual_seed(77)
    new = {x: (torch.randn((steps, N, H, d), generator=gen) * w.qk_scale if x != "v" else
               torch.randn((steps, N, H, d), generator=gen)).to(torch.bfloat16) for x in ("q", "k", "v")}
    for t in range(steps):
        o = binding.lin_attn_decode_step(new["q"][t].to(DEV), new["k"][t].to(DEV), new["v"][t].to(DEV), S,
                                         Z if normalize else None, psi=psi, normalize=normalize, eps=w.eps,
                                         gamma=gam)
        torch.cuda.synchronize()
        for b, L in enumerate(lengths):
            # the oracle over prompt b followed by generated tokens 0..t
            full = {x: torch.cat([_seq(inp[x], cu, b), new[x][:t + 1, b].transpose(0, 1)], 1).contiguous()
                    for x in ("q", "k", "v")}
            ref = _oracle_blocks(w, full["q"], full["k"], full["v"], inp, list(range(H)))
            assert_close(o[b].cpu().numpy(), ref[:, -1, :], "bf16", f"handoff seq {b} step {t}")


def test_full_varlen_serving_sampled():
    """The packed serving batch at full size (32 prompts of 1k..16k tokens, 32 heads, retention
    form), in the launch configuration the benchmark times; sampled (sequence, head) pairs
    against the oracle: the shortest, the longest and a middle sequence."""
    from chunked_causal_linear_k1_amd import workloads
    w = workloads.VARLEN_32
    announce(f"varlen full {w.name}")
    inp = inputs.make_varlen_inputs(w, device=DEV)
    g = inp["gamma"]
    o = binding.lin_attn_prefill_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["max_len"], psi=w.psi,
                                        chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=list(g))
    torch.cuda.synchronize()
    lengths = inp["lengths"]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    order = np.argsort(lengths)
    for b in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        for h in (0, w.H - 1):
            sl = slice(int(cu[b]), int(cu[b + 1]))
            q, k, v = (inp[x][sl, h].cpu().unsqueeze(0) for x in ("q", "k", "v"))
            ref = oracle.prefill(q, k, v, w.psi, gamma=[float(g[h])], normalize=w.normalize,
                                 eps=float(np.float32(w.eps)))
            assert_close(o[sl, h].cpu().unsqueeze(0).numpy(), ref, "bf16", f"varlen full seq {b} (T={lengths[b]}) head {h}")
