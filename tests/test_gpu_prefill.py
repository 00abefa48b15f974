"""GPU parity of lin_attn_prefill against the fp64 oracle (through the C ABI).

Small cases span several chunks and segments and end in a ragged chunk; they are
compared element by element. Full-size workloads are compared on every output, with the
oracle run over groups of (batch, head) sequences. Edge cases: T = 1,
T = C - 1, C, C + 1, initial/final state hand-off, causality, determinism, and an
integer-valued case whose every partial sum is exact in fp32 (bit-exact check).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from chunked_causal_linear_k1_amd import binding, inputs, workloads
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, PSI_PRF, PSI_PRF_QSHIFT, Workload

from gpu_common import announce, assert_close, compare_all_blocks, oracle_blocks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


_oracle_o = oracle_blocks


def _to_dev(inp):
    out = dict(inp)
    for key in ("q", "k", "v", "prf_w"):
        if out.get(key) is not None:
            out[key] = out[key].to(DEV)
    return out


def _run(w: Workload, inp, **kw):
    o = binding.prefill_workload(w, _to_dev(inp) if inp["q"].device.type == "cpu" else inp, **kw)
    torch.cuda.synchronize()
    return o


SMALL = [
    # name, B, H, T, d, C, psi, normalize, decay, dtype
    ("elu1_c64_ragged", 1, 2, 1000, 128, 64, PSI_ELU1, 1, "none", "bf16"),
    ("elu1_c128_ragged", 2, 1, 1000, 128, 128, PSI_ELU1, 1, "none", "bf16"),
    ("identity_decay_c128", 1, 3, 777, 128, 128, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    ("identity_decay_c64_d64", 2, 2, 530, 64, 64, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    ("elu1_decay_norm_d64_c128", 1, 2, 700, 64, 128, PSI_ELU1, 1, "const:0.99", "bf16"),
    ("elu1_decay_norm_c64", 1, 2, 1500, 128, 64, PSI_ELU1, 1, "const:0.999", "bf16"),
    ("identity_norm_nodecay", 1, 2, 333, 128, 64, PSI_IDENTITY, 0, "none", "bf16"),
    # identity features with a denominator are ill-conditioned (psi(q).Z can cross zero), so
    # the retention form is the identity case tested at C = 64, d = 128 as well
    ("identity_decay_c64_d128", 1, 3, 901, 128, 64, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    # chunks of 32 tokens (walked in 64-token steps; segments hold an even number of chunks)
    ("identity_decay_c32", 1, 3, 777, 128, 32, PSI_IDENTITY, 0, "retnet_spread", "bf16"),
    ("elu1_norm_c32_d64", 2, 2, 501, 64, 32, PSI_ELU1, 1, "const:0.99", "bf16"),
    # elu+1 with a denominator and no decay at d = 64 (shared-score kernel, single roundings)
    ("elu1_norm_nodecay_d64_c64", 1, 2, 700, 64, 64, PSI_ELU1, 1, "none", "bf16"),
    ("f32_elu1_c32", 1, 2, 300, 64, 32, PSI_ELU1, 1, "none", "f32"),
    ("f32_identity_decay_c16", 1, 2, 200, 32, 16, PSI_IDENTITY, 0, "const:0.9", "f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_elementwise(case):
    name, B, H, T, d, C, psi, normalize, decay, dt = case
    scale = (d ** -0.5) if psi == PSI_IDENTITY else 0.5
    w = Workload(name=name, B=B, H=H, T=T, d_k=d, d_v=d, n_psi=d, chunk=C, psi=psi, normalize=normalize,
                 eps=1e-6, dtype=dt, seed=11, qk_scale=scale, v_scale=1.0, decay=decay)
    announce(f"prefill small {name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(B * H, T, d).numpy(), ref, dt, name)


@pytest.mark.parametrize("d,C,decay", [(128, 128, "retnet_spread"), (128, 64, "retnet_spread"), (64, 64, "none"),
                                       (64, 128, "const:0.97")])
def test_identity_with_denominator(d, C, decay):
    """Identity features with the denominator. With signed q and k the dot psi(q).Z can pass
    through zero and the output has no bound, so here q and k are made non-negative: the
    denominator is then a positive sum and the normalised output a weighted mean of v."""
    T = 601
    w = Workload(name=f"identity_norm_d{d}_c{C}", B=1, H=3, T=T, d_k=d, d_v=d, n_psi=d, chunk=C, psi=PSI_IDENTITY,
                 normalize=1, eps=1e-6, dtype="bf16", seed=d + C, qk_scale=d ** -0.5, v_scale=1.0, decay=decay)
    announce(f"prefill identity with denominator d={d} C={C}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    inp["q"], inp["k"] = inp["q"].abs(), inp["k"].abs()
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(3, T, d).numpy(), ref, "bf16", w.name)


@pytest.mark.parametrize("d,C,decay", [(128, 64, "none"), (128, 64, "const:0.99"), (128, 128, "retnet_spread"),
                                       (64, 64, "none"), (64, 32, "const:0.99")])
def test_elu1_without_denominator(d, C, decay):
    """elu+1 features without the denominator: the unnormalised sums have no fixed scale
    (|o| reaches about 1e3 here), so rel-L2 is taken as is and max-abs on outputs scaled by
    the largest reference magnitude."""
    T = 700
    w = Workload(name=f"elu1_nonorm_d{d}_c{C}_{decay}", B=1, H=2, T=T, d_k=d, d_v=d, n_psi=d, chunk=C,
                 psi=PSI_ELU1, normalize=0, eps=1e-6, dtype="bf16", seed=d + C + 7, qk_scale=0.5, v_scale=1.0,
                 decay=decay)
    announce(f"prefill {w.name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp).cpu().reshape(2, T, d).numpy()
    ref = _oracle_o(w, inp)
    scale = float(np.abs(ref).max())
    assert_close(o / scale, ref / scale, "bf16", f"{w.name} (scaled by max |o| = {scale:.3g})")


def test_tiny_f32_workload_full():
    """The 1 x 1 x 1024, d = 64, C = 64, elu+1 fp32 workload, every output."""
    w = workloads.TINY_F32
    announce("prefill tiny_f32 full")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(1, w.T, w.d_v).numpy(), ref, "f32", w.name)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 128, 129, 191])
@pytest.mark.parametrize("C", [64, 128])
def test_edge_lengths(T, C):
    w = Workload(name=f"edge_T{T}_C{C}", B=1, H=2, T=T, d_k=128, d_v=128, n_psi=128, chunk=C, psi=PSI_ELU1,
                 normalize=1, eps=1e-6, dtype="bf16", seed=T + C, qk_scale=0.5, v_scale=1.0, decay="const:0.98")
    announce(f"prefill edge T={T} C={C}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(2, T, 128).numpy(), ref, "bf16", w.name)


def test_initial_and_final_state():
    """Prefill with an initial state equals the oracle continuing from that state; the
    final state equals the oracle's state after the last token (gamma^L for the ragged
    last chunk, not gamma^C)."""
    w = Workload(name="state", B=2, H=2, T=459, d_k=128, d_v=128, n_psi=128, chunk=128, psi=PSI_ELU1,
                 normalize=1, eps=1e-6, dtype="bf16", seed=5, qk_scale=0.5, v_scale=1.0, decay="const:0.995")
    announce("prefill init/final state")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    rng = np.random.default_rng(3)
    S0 = (rng.standard_normal((2, 2, 128, 128)) * 0.5).astype(np.float32)
    Z0 = (np.abs(rng.standard_normal((2, 2, 128))) * 10 + 1).astype(np.float32)
    fS = torch.empty((2, 2, 128, 128), dtype=torch.float32, device=DEV)
    fZ = torch.empty((2, 2, 128), dtype=torch.float32, device=DEV)
    o = _run(w, inp, init_S=torch.from_numpy(S0).to(DEV), init_Z=torch.from_numpy(Z0).to(DEV), final_S=fS,
             final_Z=fZ)
    ref, rS, rZ = _oracle_o(w, inp, S0=S0.reshape(4, 128, 128).astype(np.float64),
                            Z0=Z0.reshape(4, 128).astype(np.float64), want_state=True)
    assert_close(o.cpu().reshape(4, w.T, 128).numpy(), ref, "bf16", "o with init state")
    assert_close(fS.cpu().reshape(4, 128, 128).numpy(), rS, "bf16", "final S")
    assert_close(fZ.cpu().reshape(4, 128).numpy(), rZ, "bf16", "final Z")


def test_subsegment_records_and_final_state():
    """Enough sequences for 2048-token segments, so the summary pass folds each segment as two
    1024-token records: with a final state asked for it folds every segment; without one it
    stops at the last segment's start. Both against the oracle (sampled heads, initial state
    given, per-head decay, ragged last chunk)."""
    B, H, T, d = 2, 64, 4000, 64
    w = Workload(name="subseg", B=B, H=H, T=T, d_k=d, d_v=d, n_psi=d, chunk=64, psi=PSI_ELU1, normalize=1,
                 eps=1e-6, dtype="bf16", seed=12, qk_scale=0.5, v_scale=1.0, decay="retnet_spread")
    desc = binding.prefill_desc(B, H, T, d, d, d, 64, PSI_ELU1, 1, 1e-6, binding.LA_BF16, binding.LA_F32,
                                binding.LA_LAYOUT_BHTD)
    assert binding.workspace_size(desc) == 4 * (d * d + d) * B * H * 2 * 2  # 2 segments x 2 records
    announce("prefill sub-segment records, with and without the final state")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    rng = np.random.default_rng(9)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    Z0 = (np.abs(rng.standard_normal((B, H, d))) * 10 + 1).astype(np.float32)
    init = dict(init_S=torch.from_numpy(S0).to(DEV), init_Z=torch.from_numpy(Z0).to(DEV))
    fS = torch.empty((B, H, d, d), dtype=torch.float32, device=DEV)
    fZ = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    o_fin = _run(w, inp, final_S=fS, final_Z=fZ, **init).cpu().reshape(B * H, T, d).numpy()
    o_nof = _run(w, inp, **init).cpu().reshape(B * H, T, d).numpy()
    heads = [0, 45, 64, 127]
    ref, rS, rZ = _oracle_o(w, inp, heads=heads, S0=S0.reshape(B * H, d, d)[heads].astype(np.float64),
                            Z0=Z0.reshape(B * H, d)[heads].astype(np.float64), want_state=True)
    assert_close(o_fin[heads], ref, "bf16", "o, final state asked for")
    assert_close(o_nof[heads], ref, "bf16", "o, no final state")
    assert_close(o_nof, o_fin, "bf16", "o with and without the final state")
    assert_close(fS.cpu().reshape(B * H, d, d).numpy()[heads], rS, "bf16", "final S")
    assert_close(fZ.cpu().reshape(B * H, d).numpy()[heads], rZ, "bf16", "final Z")


@pytest.mark.parametrize("psi,decay,C", [(PSI_ELU1, "none", 64), (PSI_ELU1, "const:0.999", 64),
                                         (PSI_ELU1, "retnet_spread", 128), (PSI_ELU1, "const:0.99", 32),
                                         (PSI_PRF, "const:0.995", 64), (PSI_PRF_QSHIFT, "none", 128)])
def test_output_pass_folds_records(psi, decay, C):
    """Few sequences at d = 128 (elu+1 features with a denominator, or random features with
    n_psi 256): segments of two records each, at most six records before a segment, so with no
    initial or final state the eight-wave output pass folds the records itself (no scan), with
    the decay of each record between them. Every output against the oracle, and against the same
    call with a final state asked for (which takes the scan and, for elu+1, two-term summary
    records)."""
    B, H, T, d = 1, 2, 8000, 128
    prf = psi in (PSI_PRF, PSI_PRF_QSHIFT)
    w = Workload(name="fold", B=B, H=H, T=T, d_k=d, d_v=d, n_psi=256 if prf else d, chunk=C, psi=psi, normalize=1,
                 eps=1e-6, dtype="bf16", seed=21, qk_scale=d ** -0.25 if prf else 0.5, v_scale=0.5, decay=decay)
    announce(f"prefill output pass folding records psi={psi} decay={decay} C={C}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o_fold = _run(w, inp).cpu().reshape(B * H, T, d).numpy()
    fS = torch.empty((B, H, w.n_psi, d), dtype=torch.float32, device=DEV)
    fZ = torch.empty((B, H, w.n_psi), dtype=torch.float32, device=DEV)
    o_scan = _run(w, inp, final_S=fS, final_Z=fZ).cpu().reshape(B * H, T, d).numpy()
    ref = _oracle_o(w, inp)
    assert_close(o_fold, ref, "bf16", f"o folded records (psi {psi}, {decay}, C={C})")
    assert_close(o_scan, ref, "bf16", f"o scanned records (psi {psi}, {decay}, C={C})")
    assert_close(o_fold, o_scan, "bf16", "o folded against scanned")


def test_f32_latency_chunking():
    """An fp32 call too small to fill the GPU with its own chunks walks 16-token chunks: chunk 64
    and chunk 16 then take the same plan and give bitwise equal outputs, both at the fp32 bar."""
    w = Workload(name="f32_lat", B=1, H=2, T=700, d_k=64, d_v=64, n_psi=64, chunk=64, psi=PSI_ELU1, normalize=1,
                 eps=1e-6, dtype="f32", seed=31, qk_scale=0.5, v_scale=1.0, decay="const:0.99")
    announce("prefill fp32 latency chunking")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o64 = _run(w, inp).cpu().numpy()
    o16 = _run(dataclasses.replace(w, chunk=16), inp).cpu().numpy()
    assert np.array_equal(o64, o16), "chunk 64 and chunk 16 took different plans"
    assert_close(o64.reshape(2, w.T, 64), _oracle_o(w, inp), "f32", "o, fp32 latency chunking")


def test_initial_and_final_state_c64():
    """The same hand-off at C = 64 (the two-waves-per-SIMD output kernel), per-head decay."""
    w = Workload(name="state_c64", B=2, H=3, T=777, d_k=128, d_v=128, n_psi=128, chunk=64, psi=PSI_ELU1,
                 normalize=1, eps=1e-6, dtype="bf16", seed=6, qk_scale=0.5, v_scale=1.0, decay="retnet_spread")
    announce("prefill init/final state C=64")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    rng = np.random.default_rng(8)
    S0 = (rng.standard_normal((2, 3, 128, 128)) * 0.5).astype(np.float32)
    Z0 = (np.abs(rng.standard_normal((2, 3, 128))) * 10 + 1).astype(np.float32)
    fS = torch.empty((2, 3, 128, 128), dtype=torch.float32, device=DEV)
    fZ = torch.empty((2, 3, 128), dtype=torch.float32, device=DEV)
    o = _run(w, inp, init_S=torch.from_numpy(S0).to(DEV), init_Z=torch.from_numpy(Z0).to(DEV), final_S=fS,
             final_Z=fZ)
    ref, rS, rZ = _oracle_o(w, inp, S0=S0.reshape(6, 128, 128).astype(np.float64),
                            Z0=Z0.reshape(6, 128).astype(np.float64), want_state=True)
    assert_close(o.cpu().reshape(6, w.T, 128).numpy(), ref, "bf16", "o with init state, C=64")
    assert_close(fS.cpu().reshape(6, 128, 128).numpy(), rS, "bf16", "final S, C=64")
    assert_close(fZ.cpu().reshape(6, 128).numpy(), rZ, "bf16", "final Z, C=64")


def test_causality_and_determinism():
    w = Workload(name="causal", B=1, H=2, T=700, d_k=128, d_v=128, n_psi=128, chunk=64, psi=PSI_ELU1,
                 normalize=1, eps=1e-6, dtype="bf16", seed=9, qk_scale=0.5, v_scale=1.0)
    announce("prefill causality/determinism")
    inp = _to_dev(inputs.make_prefill_inputs(w, device="cpu"))
    o1 = _run(w, inp).clone()
    o2 = _run(w, inp).clone()
    assert torch.equal(o1, o2), "two identical calls differ"
    t0 = 333
    inp2 = dict(inp)
    for key in ("q", "k", "v"):
        x = inp[key].clone()
        x[:, :, t0:] = -x[:, :, t0:] + 0.25
        inp2[key] = x
    o3 = _run(w, inp2)
    # outputs before t0 only depend on tokens before t0; chunks that straddle t0 use the
    # same arithmetic for those rows, so they are bitwise unchanged as well
    assert torch.equal(o1[:, :, :t0], o3[:, :, :t0])
    assert not torch.equal(o1[:, :, t0:], o3[:, :, t0:])


def test_integer_inputs_bit_exact():
    """gamma = 1, identity psi, no denominator, entries in {-1, 0, 1}, d = 64, T = 1000:
    every product and partial sum is an integer below 2^24, so fp32 accumulation is exact
    and the GPU must equal the oracle bit for bit, through the scan and the ragged tail."""
    for C in (64, 128):
        announce(f"prefill integer exact C={C}")
        ints = inputs.small_integer_inputs(1, 2, 1000, 64, 64, -1, 1, seed=C)
        w = Workload(name="int", B=1, H=2, T=1000, d_k=64, d_v=64, n_psi=64, chunk=C, psi=PSI_IDENTITY,
                     normalize=0, eps=0.0, dtype="bf16", seed=0, qk_scale=1.0, v_scale=1.0)
        inp = {"q": ints["q"], "k": ints["k"], "v": ints["v"], "gamma": None, "prf_w": None}
        o = _run(w, inp)
        ref = _oracle_o(w, inp)
        np.testing.assert_array_equal(o.cpu().reshape(2, 1000, 64).numpy().astype(np.float64), ref)


def test_chunk_size_invariance():
    """C = 32, 64 and 128 compute the same function: each within tolerance of the oracle
    and of C = 64."""
    base = dict(B=1, H=2, T=900, d_k=128, d_v=128, n_psi=128, psi=PSI_IDENTITY, normalize=0, eps=1e-6,
                dtype="bf16", seed=21, qk_scale=128 ** -0.5, v_scale=1.0, decay="retnet_spread")
    announce("prefill chunk-size invariance")
    w64 = Workload(name="c64", chunk=64, **base)
    w128 = Workload(name="c128", chunk=128, **base)
    inp = inputs.make_prefill_inputs(w64, device="cpu")
    o64 = _run(w64, inp).cpu().numpy()
    o128 = _run(w128, inp).cpu().numpy()
    o32 = _run(Workload(name="c32", chunk=32, **base), inp).cpu().numpy()
    ref = _oracle_o(w64, inp)
    assert_close(o64.reshape(2, 900, 128), ref, "bf16", "C=64")
    assert_close(o128.reshape(2, 900, 128), ref, "bf16", "C=128")
    assert_close(o32.reshape(2, 900, 128), ref, "bf16", "C=32")
    assert_close(o64, o128, "bf16", "C=64 vs C=128")
    assert_close(o64, o32, "bf16", "C=64 vs C=32")


def _full_size(w: Workload):
    """Every output of a full-size workload, in the launch configuration the benchmark times
    (inputs drawn on the GPU, default layout, fp32 output), against the oracle."""
    announce(f"prefill full-size {w.name}, all {w.B * w.H} (batch, head) blocks")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    o = binding.prefill_workload(w, inp)
    torch.cuda.synchronize()
    compare_all_blocks(w, o, inp, w.name)


def test_full_prefill_8k_elu1():
    _full_size(workloads.PREFILL_8K)


def test_full_retnet_128k():
    _full_size(workloads.RETNET_128K)


def test_context_parallel_share_128k():
    """One GPU's view of context parallelism on the 128k retention workload (the method's scan
    lifted to contiguous T-shards, one per GPU): T is cut into 8 shards; each shard's summary is
    its final state from a zero initial state, computed independently; the summaries are folded
    in rank order under the decayed monoid (P_{r+1} = gamma^{L_r} P_r + S_r, what every GPU does
    after gathering them); and each shard's prefill then starts from its predecessors' fold.
    Concatenated, the shard outputs must equal the single call's to fp32 rounding, and sampled
    heads must match the oracle."""
    w = workloads.RETNET_128K
    announce("context-parallel share: 128k retention in 8 T-shards")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    o_full = binding.prefill_workload(w, inp)
    gam = torch.tensor(np.asarray(inp["gamma"], dtype=np.float64), device=DEV)  # the fp32 values, exactly
    P = 8
    bounds = [r * 16384 for r in range(P)] + [w.T]
    shards = [{key: inp[key][:, :, lo:hi].contiguous() for key in ("q", "k", "v")}
              for lo, hi in zip(bounds[:-1], bounds[1:])]
    g = list(inp["gamma"])
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=0, eps=w.eps, gamma=g)
    summaries = []
    for sh in shards:  # independent: each shard alone from a zero state
        fS = torch.empty((1, w.H, 128, 128), device=DEV)
        binding.lin_attn_prefill(sh["q"], sh["k"], sh["v"], final_S=fS, **kw)
        summaries.append(fS)
    torch.cuda.synchronize()
    prefix = torch.zeros((1, w.H, 128, 128), dtype=torch.float64, device=DEV)
    outs = []
    for r, sh in enumerate(shards):
        outs.append(binding.lin_attn_prefill(sh["q"], sh["k"], sh["v"], init_S=prefix.float().contiguous(), **kw))
        L = bounds[r + 1] - bounds[r]
        prefix = (gam ** L).view(1, w.H, 1, 1) * prefix + summaries[r].double()
    torch.cuda.synchronize()
    o_sh = torch.cat(outs, dim=2)
    rel = float((o_sh.double() - o_full.double()).norm() / o_full.double().norm())
    print(f"[parity] sharded vs single call rel_l2={rel:.3e}", flush=True)
    assert rel <= 1e-5, rel
    heads = [0, 63]
    ref = _oracle_o(w, inp, heads=heads)
    assert_close(o_sh.reshape(w.H, w.T, w.d_v)[heads].cpu().numpy(), ref, "bf16", "sharded 128k heads 0, 63")


# positive random features (psi = exp(W x - |x|^2/2) / sqrt(n_psi), one bf16 bank per head)
PRF_SMALL = [
    # name, B, H, T, n_psi, normalize, decay, v_scale
    ("prf256_ragged", 1, 2, 450, 256, 1, "none", 1.0),
    ("prf128_ragged", 2, 1, 333, 128, 1, "none", 1.0),
    ("prf256_decay_norm", 1, 2, 400, 256, 1, "const:0.99", 1.0),
    ("prf128_decay_norm_spread", 1, 3, 260, 128, 1, "retnet_spread", 1.0),
    ("prf256_decay_nonorm", 1, 2, 300, 256, 0, "retnet_spread", 0.05),
]


@pytest.mark.parametrize("case", PRF_SMALL, ids=[c[0] for c in PRF_SMALL])
def test_prf_small_elementwise(case):
    name, B, H, T, n_psi, normalize, decay, vs = case
    w = Workload(name=name, B=B, H=H, T=T, d_k=128, d_v=128, n_psi=n_psi, chunk=64, psi=PSI_PRF,
                 normalize=normalize, eps=1e-6, dtype="bf16", seed=13, qk_scale=128 ** -0.25, v_scale=vs,
                 decay=decay)
    announce(f"prefill prf small {name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp).cpu().reshape(B * H, T, 128).numpy()
    ref = _oracle_o(w, inp)
    if normalize:
        assert_close(o, ref, "bf16", name)
    else:
        # unnormalised sums of exponential features have no fixed scale (here |o| ~ 1e3):
        # rel-L2 as is, max-abs on outputs scaled by the largest reference magnitude
        scale = float(np.abs(ref).max())
        assert_close(o / scale, ref / scale, "bf16", f"{name} (scaled by max |o| = {scale:.3g})")


@pytest.mark.parametrize("C", [32, 128])
def test_prf_chunk_sizes(C):
    """Positive random features with chunks of 32 and 128 tokens (the kernels' 64-token steps)."""
    w = Workload(name=f"prf256_c{C}", B=1, H=2, T=450, d_k=128, d_v=128, n_psi=256, chunk=C, psi=PSI_PRF,
                 normalize=1, eps=1e-6, dtype="bf16", seed=17, qk_scale=128 ** -0.25, v_scale=1.0,
                 decay="const:0.99")
    announce(f"prefill prf chunk {C}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp).cpu().reshape(2, 450, 128).numpy()
    assert_close(o, _oracle_o(w, inp), "bf16", f"prf chunk {C}")


# the same features with the query-row log-space shift (psi(q)_p = exp(l_p - max_r l_r) / sqrt(m))
PRF_QSHIFT = [
    # name, T, n_psi, normalize, decay, query multiplier
    ("qshift256", 450, 256, 1, "none", 1.0),
    ("qshift128_decay", 333, 128, 1, "const:0.99", 1.0),
    # queries 8x larger: unshifted log-features near -300 underflow in fp32, shifted ones peak at 0
    ("qshift256_large_queries", 400, 256, 1, "none", 8.0),
    ("qshift128_large_queries_decay", 200, 128, 1, "const:0.98", 8.0),
]


@pytest.mark.parametrize("case", PRF_QSHIFT, ids=[c[0] for c in PRF_QSHIFT])
def test_prf_qshift(case):
    name, T, n_psi, normalize, decay, q_mult = case
    B, H = 1, 2
    w = Workload(name=name, B=B, H=H, T=T, d_k=128, d_v=128, n_psi=n_psi, chunk=64, psi=PSI_PRF_QSHIFT,
                 normalize=normalize, eps=1e-6, dtype="bf16", seed=19, qk_scale=128 ** -0.25, v_scale=1.0,
                 decay=decay)
    announce(f"prefill prf query shift {name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    inp["q"] = (inp["q"].float() * q_mult).to(torch.bfloat16)  # a power of two: exact
    o = _run(w, inp).cpu().reshape(B * H, T, 128).numpy()
    assert_close(o, _oracle_o(w, inp), "bf16", name)


def test_prf_qshift_without_denominator_is_refused():
    """The shift cancels only against the denominator, so normalize = 0 is refused before launch."""
    w = Workload(name="qshift_nonorm", B=1, H=2, T=64, d_k=128, d_v=128, n_psi=256, chunk=64, psi=PSI_PRF_QSHIFT,
                 normalize=0, eps=1e-6, dtype="bf16", seed=19, qk_scale=128 ** -0.25, v_scale=1.0)
    inp = inputs.make_prefill_inputs(w, device="cpu")
    with pytest.raises(binding.LinAttnError) as e:
        _run(w, inp)
    assert e.value.status == binding.LA_ERR_UNSUPPORTED


@pytest.mark.parametrize("psi", [PSI_PRF, PSI_PRF_QSHIFT])
def test_prf_orthogonal_bank(psi):
    """The orthogonal Gaussian bank ("Linearized 2-Simplicial Attention", appendix B.1: Haar
    blocks of 128 rows with chi_128 radii) in place of the independent one."""
    from chunked_causal_linear_k1_amd import prf_bank
    w = Workload(name="prf_orthogonal", B=1, H=2, T=350, d_k=128, d_v=128, n_psi=256, chunk=64, psi=psi,
                 normalize=1, eps=1e-6, dtype="bf16", seed=29, qk_scale=128 ** -0.25, v_scale=1.0,
                 decay="const:0.995")
    announce(f"prefill prf orthogonal bank psi={psi}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    inp["prf_w"] = prf_bank.orthogonal_bank(2, 256, 128, seed=5)
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(2, 350, 128).numpy(), ref, "bf16", f"orthogonal bank psi={psi}")


def test_prf_qshift_f32_path():
    """The fp32 path with the query-row shift (d 64, n_psi 96, chunk 32)."""
    w = Workload(name="f32_qshift", B=1, H=2, T=150, d_k=64, d_v=64, n_psi=96, chunk=32, psi=PSI_PRF_QSHIFT,
                 normalize=1, eps=1e-6, dtype="f32", seed=23, qk_scale=64 ** -0.25, v_scale=1.0,
                 decay="const:0.97")
    announce("prefill prf query shift fp32")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp).cpu().reshape(2, 150, 64).numpy()
    ref = _oracle_o(w, inp)
    assert_close(o, ref, "f32", w.name)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_prf_edge_lengths(T):
    w = Workload(name=f"prf_edge_T{T}", B=1, H=2, T=T, d_k=128, d_v=128, n_psi=256, chunk=64, psi=PSI_PRF,
                 normalize=1, eps=1e-6, dtype="bf16", seed=40 + T, qk_scale=128 ** -0.25, v_scale=1.0)
    announce(f"prefill prf edge T={T}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(2, T, 128).numpy(), ref, "bf16", w.name)


def test_prf_initial_and_final_state():
    """n_psi = 256 != d_v: the 256 x 128 state and 256-long normaliser in and out."""
    B, H, T, NP = 1, 2, 301, 256
    w = Workload(name="prf_state", B=B, H=H, T=T, d_k=128, d_v=128, n_psi=NP, chunk=64, psi=PSI_PRF,
                 normalize=1, eps=1e-6, dtype="bf16", seed=17, qk_scale=128 ** -0.25, v_scale=1.0,
                 decay="const:0.995")
    announce("prefill prf init/final state")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    rng = np.random.default_rng(4)
    S0 = (rng.standard_normal((B, H, NP, 128)) * 0.5).astype(np.float32)
    Z0 = (np.abs(rng.standard_normal((B, H, NP))) * 5 + 1).astype(np.float32)
    fS = torch.empty((B, H, NP, 128), dtype=torch.float32, device=DEV)
    fZ = torch.empty((B, H, NP), dtype=torch.float32, device=DEV)
    o = _run(w, inp, init_S=torch.from_numpy(S0).to(DEV), init_Z=torch.from_numpy(Z0).to(DEV), final_S=fS,
             final_Z=fZ)
    ref, rS, rZ = _oracle_o(w, inp, S0=S0.reshape(B * H, NP, 128).astype(np.float64),
                            Z0=Z0.reshape(B * H, NP).astype(np.float64), want_state=True)
    assert_close(o.cpu().reshape(B * H, T, 128).numpy(), ref, "bf16", "prf o with init state")
    assert_close(fS.cpu().reshape(B * H, NP, 128).numpy() / np.abs(rS).max(), rS / np.abs(rS).max(), "bf16",
                 "prf final S (scaled to max 1)")
    assert_close(fZ.cpu().reshape(B * H, NP).numpy() / np.abs(rZ).max(), rZ / np.abs(rZ).max(), "bf16",
                 "prf final Z (scaled to max 1)")


STRONG_DECAY = [
    # name, psi, normalize, d, n_psi, decay: gamma far below 1, where gamma^n for the padded rows of
    # a ragged last chunk (n < 0) would overflow fp32
    ("identity_g0.1", PSI_IDENTITY, 0, 128, 128, "const:0.1"),
    ("elu1_norm_g0.05", PSI_ELU1, 1, 128, 128, "const:0.05"),
    ("elu1_norm_g0.1_d64", PSI_ELU1, 1, 64, 64, "const:0.1"),
    ("prf256_norm_g0.1", PSI_PRF, 1, 128, 256, "const:0.1"),
]


@pytest.mark.parametrize("case", STRONG_DECAY, ids=[c[0] for c in STRONG_DECAY])
def test_strong_decay_ragged_final_state(case):
    """Strong decay, a ragged last chunk and the final state asked for: the padded rows' decay
    factors are never formed, so outputs and the final state stay finite and match the oracle."""
    name, psi, norm, d, NP, decay = case
    B, H, T = 1, 2, 2 * 2048 + 1  # one real token in the last 64-token step: 63 padded rows
    qks = {PSI_IDENTITY: d ** -0.5, PSI_ELU1: 0.5, PSI_PRF: d ** -0.25}[psi]
    w = Workload(name=f"strong_{name}", B=B, H=H, T=T, d_k=d, d_v=d, n_psi=NP, chunk=64, psi=psi, normalize=norm,
                 eps=1e-6, dtype="bf16", seed=41, qk_scale=qks, v_scale=1.0, decay=decay)
    announce(f"prefill strong decay {name}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    fS = torch.empty((B, H, NP, d), dtype=torch.float32, device=DEV)
    fZ = torch.empty((B, H, NP), dtype=torch.float32, device=DEV)
    o = _run(w, inp, final_S=fS, final_Z=fZ)
    ref, rS, rZ = _oracle_o(w, inp, want_state=True)
    assert torch.isfinite(o).all() and torch.isfinite(fS).all(), name
    assert_close(o.cpu().reshape(B * H, T, d).numpy(), ref, "bf16", f"{name} o")
    assert_close(fS.cpu().reshape(B * H, NP, d).numpy() / np.abs(rS).max(), rS / np.abs(rS).max(), "bf16",
                 f"{name} final S (scaled to max 1)")
    if norm:
        assert torch.isfinite(fZ).all(), name
        assert_close(fZ.cpu().reshape(B * H, NP).numpy() / np.abs(rZ).max(), rZ / np.abs(rZ).max(), "bf16",
                     f"{name} final Z (scaled to max 1)")


def test_full_prf_4k():
    _full_size(workloads.PRF_4K)


def test_full_prf_4k_qshift():
    """The PRF workload with the query-row shift, every output."""
    _full_size(workloads.PRF_4K.with_(name="prf256_4k_qshift", psi=PSI_PRF_QSHIFT))


def test_max_decay_heads():
    """LA_MAX_DECAY_HEADS = 256 heads, each with its own decay (the spread formula over 256 heads),
    every head against the oracle: the largest per-head table the launch arguments carry."""
    w = Workload(name="decay256", B=1, H=256, T=200, d_k=64, d_v=64, n_psi=64, chunk=64, psi=PSI_IDENTITY,
                 normalize=0, eps=1e-6, dtype="bf16", seed=41, qk_scale=64 ** -0.5, v_scale=1.0,
                 decay="retnet_spread")
    announce("prefill 256 decayed heads")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    assert len(set(np.asarray(inp["gamma"]).tolist())) > 200  # distinct decays
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(w.H, w.T, w.d_v).numpy(), ref, "bf16", "256 decayed heads")


def test_more_sequences_than_65535():
    """B x H beyond 65535 (the y extent of a grid): sequences sit on the grid's x extent in
    every pass (summaries, scan, outputs), so 70000 short sequences (T = 40: a full chunk
    and a ragged one) are computed like any others. Every output is compared with the
    oracle."""
    w = Workload(name="many_sequences", B=70000, H=1, T=40, d_k=64, d_v=64, n_psi=64, chunk=32, psi=PSI_ELU1,
                 normalize=1, eps=1e-6, dtype="bf16", seed=17, qk_scale=0.5, v_scale=1.0)
    announce("prefill 70000 sequences of 70 tokens")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    o = _run(w, inp)
    ref = _oracle_o(w, inp)
    assert_close(o.cpu().reshape(w.B * w.H, w.T, w.d_v).numpy(), ref, "bf16", w.name)


@pytest.mark.parametrize("n_seg", [1, 2, 3, 4, 5, 8, 16, 17, 64, 65, 100, 128, 129, 256, 257, 600, 1024, 1025, 4096,
                                   65535])
def test_scan_depth_record(n_seg):
    """The segment scan's depth as the kernel counts it while it runs ("Log-Depth Chunked
    Linear-Attention Scan", Verification: the round count is the check of the scan's depth),
    and its result. Up to 128 segments, W waves (a power of two, at most 16, about 4
    segments each) fold their runs in sequence, a Blelloch tree over the W totals takes
    log2 W levels up and log2 W down, one step carries the initial state and each run is
    rewritten: 2 ceil(n / W) + 2 log2 W + 1 levels, at most 17 up to 64 segments. Beyond 128
    the lanes hold segments: per block of 64 NW segments, 6 rounds of lane shifts
    (Hillis-Steele across a wavefront), log2 NW levels up and down across the waves
    (Blelloch) and 2 combines with the carried prefix: ceil(n / (64 NW)) (8 + 2 log2 NW), 16
    levels for 1024 segments. Integer-valued records make every prefix exact in fp32, so the
    exclusive prefixes must equal the host's cumulative sums bit for bit."""
    if n_seg <= 128:
        W = 1
        while W < 16 and W * 4 < n_seg:
            W *= 2
        want = 2 * (-(-n_seg // W)) + 2 * (W.bit_length() - 1) + 1
    else:
        NW = 4 if n_seg <= 256 else 8 if n_seg <= 512 else 16
        want = (-(-n_seg // (64 * NW))) * (8 + 2 * (NW.bit_length() - 1))
    announce(f"scan depth n_seg={n_seg}")
    gen = torch.Generator().manual_seed(n_seg)
    rec = torch.randint(-8, 9, (n_seg, 20), generator=gen).to(torch.float32)
    got, pre = binding.scan_depth(n_seg, rec)
    print(f"[scan depth] n_seg={n_seg} rounds={got} (ceil(log2 n) = {(n_seg - 1).bit_length()})", flush=True)
    assert got == want
    if n_seg <= 64:
        assert got <= 17
    ref = torch.cumsum(rec.double(), 0) - rec.double()
    assert torch.equal(pre.cpu().double(), ref)


@pytest.mark.parametrize("psi,decay", [(PSI_IDENTITY, "retnet_spread"), (PSI_ELU1, "const:0.9995")])
def test_long_sequence_many_segments(psi, decay):
    """A sequence long enough for more than 128 segments (300,000 tokens: 247 segments of
    1216 tokens), so the segment scan runs its many-segment form (lanes over segments), with
    an initial state handed in and the final state taken out. Every output and the final
    state are compared with the oracle."""
    normalize = 1 if psi == PSI_ELU1 else 0
    w = Workload(name="long_many_segments", B=1, H=1, T=300000, d_k=64, d_v=64, n_psi=64, chunk=64, psi=psi,
                 normalize=normalize, eps=1e-6, dtype="bf16", seed=29, qk_scale=(64 ** -0.5) if psi == PSI_IDENTITY else 0.5,
                 v_scale=1.0, decay=decay)
    announce(f"prefill long sequence psi={psi} T={w.T}")
    inp = inputs.make_prefill_inputs(w, device="cpu")
    gen = torch.Generator().manual_seed(31)
    S0 = (torch.randn((1, 1, 64, 64), generator=gen) * 0.1).float()
    Z0 = (torch.rand((1, 1, 64), generator=gen) + 0.5).float()
    fS = torch.empty((1, 1, 64, 64), device=DEV)
    fZ = torch.empty((1, 1, 64), device=DEV)
    dinp = _to_dev(inp)
    o = binding.lin_attn_prefill(dinp["q"], dinp["k"], dinp["v"], psi=psi, chunk=64, normalize=normalize, eps=w.eps,
                                 gamma=None if inp["gamma"] is None else list(inp["gamma"]), init_S=S0.to(DEV),
                                 init_Z=Z0.to(DEV) if normalize else None, final_S=fS,
                                 final_Z=fZ if normalize else None)
    torch.cuda.synchronize()
    ref, rS, rZ = oracle_blocks(w, inp, S0=S0.double().numpy().reshape(1, 64, 64),
                                Z0=Z0.double().numpy().reshape(1, 64) if normalize else None, want_state=True)
    assert_close(o.cpu().reshape(1, w.T, 64).numpy(), ref, "bf16", "long sequence outputs")
    sref = rS.reshape(1, 64, 64)
    rel = float(np.linalg.norm(fS.cpu().double().numpy().reshape(1, 64, 64) - sref) / np.linalg.norm(sref))
    print(f"[parity] long sequence final S rel_l2={rel:.3e}", flush=True)
    assert rel <= 2e-3

