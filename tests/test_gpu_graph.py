"""HIP graph capture of the C ABI calls (torch.cuda.CUDAGraph): lin_attn_prefill (workspace and
no-allocation entry points), lin_attn_prefill_gated and lin_attn_decode_step recorded once and
replayed. Before each replay, eager work writes new inputs into the captured buffers; each
replay's output (and, for decode, the state it updates in place) must equal, bit for bit, an
eager call on the same inputs. The calls only enqueue kernels on the caller's stream: no
allocation, no synchronisation and no memset nodes in what they record."""
from __future__ import annotations

import pytest
import torch

from chunked_causal_linear_k1_amd import binding, inputs
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, PSI_PRF, DecodeWorkload, Workload

from gpu_common import announce

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _capture(fn) -> torch.cuda.CUDAGraph:
    """Record fn into a graph; one eager call on the side stream first (one-time set-up such as
    kernel attributes and the scratch address happens outside the capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


PREFILL = [
    Workload(name="graph_elu1_norm", B=2, H=3, T=1000, d_k=128, d_v=128, n_psi=128, chunk=64, psi=PSI_ELU1,
             normalize=1, eps=1e-6, dtype="bf16", seed=61, qk_scale=0.5, v_scale=1.0),
    Workload(name="graph_retention_c128", B=1, H=4, T=777, d_k=128, d_v=128, n_psi=128, chunk=128, psi=PSI_IDENTITY,
             normalize=0, eps=1e-6, dtype="bf16", seed=62, qk_scale=128 ** -0.5, v_scale=1.0, decay="retnet_spread"),
    Workload(name="graph_prf256", B=1, H=2, T=450, d_k=128, d_v=128, n_psi=256, chunk=64, psi=PSI_PRF, normalize=1,
             eps=1e-6, dtype="bf16", seed=63, qk_scale=128 ** -0.25, v_scale=1.0),
    Workload(name="graph_f32_elu1", B=1, H=2, T=300, d_k=64, d_v=64, n_psi=64, chunk=32, psi=PSI_ELU1, normalize=1,
             eps=1e-6, dtype="f32", seed=64, qk_scale=0.5, v_scale=1.0, decay="const:0.99"),
]


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("w", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_graph_replays(w: Workload, noalloc: bool):
    if noalloc and w.dtype != "bf16":
        pytest.skip("the no-allocation entry point serves the bf16 path")
    announce(f"graph prefill {w.name} ({'noalloc' if noalloc else 'workspace'})")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    q, k, v, prf = inp["q"], inp["k"], inp["v"], inp["prf_w"]
    g = inp["gamma"]
    args = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g),
                prf_w=prf)
    o = torch.empty((w.B, w.H, w.T, w.d_v), dtype=torch.float32, device=DEV)
    fS = torch.empty((w.B, w.H, w.n_psi, w.d_v), dtype=torch.float32, device=DEV)
    if noalloc:
        def call():
            binding.lin_attn_prefill_noalloc(q, k, v, o=o, final_S=fS, **args)
    else:
        desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                    binding.LA_BF16 if w.dtype == "bf16" else binding.LA_F32)
        ws = torch.empty(max(binding.workspace_size(desc), 16), dtype=torch.uint8, device=DEV)

        def call():
            binding.lin_attn_prefill(q, k, v, o=o, final_S=fS, workspace=ws, **args)
    graph = _capture(call)
    for rep in range(REPLAYS):
        new = inputs.make_prefill_inputs(w, device=DEV, seed=w.seed + 100 + rep)
        for dst, key in ((q, "q"), (k, "k"), (v, "v")):
            dst.copy_(new[key])
        o.fill_(float("nan"))
        graph.replay()
        fS_ref = torch.empty_like(fS)
        ref = binding.lin_attn_prefill(q, k, v, final_S=fS_ref, **args)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"{w.name}: replay {rep} differs from the eager call"
        assert torch.equal(fS, fS_ref), f"{w.name}: replay {rep} final state differs from the eager call"


def test_gated_prefill_graph_replays():
    w = Workload(name="graph_gated", B=1, H=2, T=500, d_k=128, d_v=128, n_psi=128, chunk=32, psi=PSI_IDENTITY,
                 normalize=0, eps=1e-6, dtype="bf16", seed=65, qk_scale=128 ** -0.5, v_scale=1.0)
    announce("graph gated prefill")
    inp = inputs.make_prefill_inputs(w, device=DEV)
    q, k, v = inp["q"], inp["k"], inp["v"]
    lg = inputs.make_log_gates((w.B, w.H, w.T, w.d_k), seed=66, device=DEV)
    o = torch.empty((w.B, w.H, w.T, w.d_v), dtype=torch.float32, device=DEV)
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_BF16)
    ws = torch.empty(max(binding.gated_workspace_size(desc), 16), dtype=torch.uint8, device=DEV)
    args = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps)
    graph = _capture(lambda: binding.lin_attn_prefill_gated(q, k, v, lg, o=o, workspace=ws, **args))
    for rep in range(REPLAYS):
        new = inputs.make_prefill_inputs(w, device=DEV, seed=w.seed + 100 + rep)
        for dst, key in ((q, "q"), (k, "k"), (v, "v")):
            dst.copy_(new[key])
        lg.copy_(inputs.make_log_gates(lg.shape, seed=200 + rep, device=DEV))
        o.fill_(float("nan"))
        graph.replay()
        ref = binding.lin_attn_prefill_gated(q, k, v, lg, **args)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"gated: replay {rep} differs from the eager call"


def test_decode_graph_replays():
    """One decode step captured; each replay is the next token of every stream (new q, k, v
    copied in eagerly), the state updated in place. The eager run steps its own copy of the
    starting state through the same tokens."""
    w = DecodeWorkload(name="graph_decode", N=4, H=8, d_k=128, d_v=128, n_psi=128, psi=PSI_ELU1, normalize=1,
                       eps=1e-6, gamma=0.999, prefix_len=64, steps=REPLAYS, seed=67)
    announce("graph decode step")
    prefix = inputs.make_decode_prefix(w, device=DEV)
    S = torch.empty((w.N, w.H, w.n_psi, w.d_v), dtype=torch.float32, device=DEV)
    Z = torch.empty((w.N, w.H, w.n_psi), dtype=torch.float32, device=DEV)
    gam = [w.gamma] * w.H
    binding.lin_attn_prefill(torch.zeros_like(prefix["k"]), prefix["k"], prefix["v"], psi=w.psi, chunk=64,
                             normalize=w.normalize, eps=w.eps, gamma=gam, final_S=S, final_Z=Z)
    steps = inputs.make_decode_steps(w, device=DEV)
    q, k, v = (torch.empty_like(steps[n][0]) for n in ("q", "k", "v"))
    o = torch.empty((w.N, w.H, w.d_v), dtype=torch.float32, device=DEV)
    args = dict(psi=w.psi, normalize=w.normalize, eps=w.eps, gamma=gam)
    S_ref, Z_ref = S.clone(), Z.clone()
    q.copy_(steps["q"][0]), k.copy_(steps["k"][0]), v.copy_(steps["v"][0])
    # the capture's own warm-up call is a step: the eager reference takes the same step
    graph = _capture(lambda: binding.lin_attn_decode_step(q, k, v, S, Z, o=o, **args))
    binding.lin_attn_decode_step(q, k, v, S_ref, Z_ref, **args)
    for t in range(REPLAYS):
        for dst, n in ((q, "q"), (k, "k"), (v, "v")):
            dst.copy_(steps[n][t])
        o.fill_(float("nan"))
        graph.replay()
        ref = binding.lin_attn_decode_step(q, k, v, S_ref, Z_ref, **args)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), f"decode: replay {t} output differs from the eager step"
        assert torch.equal(S, S_ref) and torch.equal(Z, Z_ref), f"decode: replay {t} state differs"
