"""lin_attn_prefill_noalloc (the prefill for callers that cannot allocate device memory) against
lin_attn_prefill through the C ABI: two calls in a row, the second smaller, each equal to the
workspace entry point's output; a call whose records exceed the scratch (fewer, longer segments)
within the bf16 bar of it and of the oracle; and a call that cannot fit refused on the host."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from chunked_causal_linear_k1_amd import binding, inputs, workloads
from chunked_causal_linear_k1_amd.workloads import PSI_ELU1, PSI_IDENTITY, Workload

from gpu_common import announce, assert_close, oracle_blocks

DEV = "cuda:0"


def _both(w: Workload, inp, **kw):
    g = inp["gamma"]
    args = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g),
                prf_w=inp.get("prf_w"), **kw)
    ref = binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], **args)
    o = torch.full_like(ref, float("nan"))
    got = binding.lin_attn_prefill_noalloc(inp["q"], inp["k"], inp["v"], o=o, **args)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.gpu
def test_noalloc_two_calls_second_smaller():
    big = Workload(name="noalloc_big", B=2, H=4, T=5000, d_k=128, d_v=128, n_psi=128, chunk=64, psi=PSI_ELU1,
                   normalize=1, eps=1e-6, dtype="bf16", seed=51, qk_scale=0.5, v_scale=1.0, decay="const:0.999")
    small = Workload(name="noalloc_small", B=1, H=3, T=777, d_k=128, d_v=128, n_psi=128, chunk=128,
                     psi=PSI_IDENTITY, normalize=0, eps=1e-6, dtype="bf16", seed=52, qk_scale=128 ** -0.5,
                     v_scale=1.0, decay="retnet_spread")
    for w in (big, small):
        announce(f"noalloc {w.name}")
        inp = inputs.make_prefill_inputs(w, device=DEV)
        fS = torch.empty((w.B, w.H, 128, 128), dtype=torch.float32, device=DEV)
        fS2 = torch.empty_like(fS)
        got, ref = _both(w, inp)
        # the same plan as the workspace entry point (its records fit the scratch): same bits
        assert torch.equal(got, ref), w.name
        assert_close(got.cpu().reshape(w.B * w.H, w.T, 128).numpy(), oracle_blocks(w, inp), "bf16", w.name)
        # with the final state as well
        g = inp["gamma"]
        args = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g))
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], final_S=fS, **args)
        binding.lin_attn_prefill_noalloc(inp["q"], inp["k"], inp["v"], final_S=fS2, **args)
        torch.cuda.synchronize()
        assert torch.equal(fS, fS2), w.name


@pytest.mark.gpu
def test_noalloc_records_beyond_scratch():
    """The 128k retention workload: its usual plan's records (about 135 MB) exceed the 64 MiB
    scratch, so the call takes fewer, longer segments; the output stays within the bf16 bar of
    the workspace entry point's, and of the oracle on sampled heads."""
    w = workloads.RETNET_128K
    announce("noalloc 128k retention (records beyond the scratch)")
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_BF16)
    assert binding.workspace_size(desc) > binding.NOALLOC_SCRATCH_BYTES
    inp = inputs.make_prefill_inputs(w, device=DEV)
    got, ref = _both(w, inp)
    rel = float((got.double() - ref.double()).norm() / ref.double().norm())
    mx = float((got - ref).abs().max())
    print(f"[parity] noalloc vs workspace call rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= 2e-3 and mx <= 1e-2
    heads = [0, 63]
    assert_close(got.reshape(w.H, w.T, w.d_v)[heads].cpu().numpy(), oracle_blocks(w, inp, heads=heads), "bf16",
                 "noalloc 128k heads 0, 63")


def test_noalloc_refuses_what_cannot_fit():
    """One record per sequence must fit the scratch: 1024 heads of d = 128 need 66 KB each, more
    than 64 MiB in all, so the call is refused before the device is touched (no GPU needed)."""
    import ctypes
    lib = binding.load()
    fake = ctypes.c_void_p(1 << 20)
    desc = binding.prefill_desc(1, 1024, 4096, 128, 128, 128, 64, PSI_IDENTITY, 0, 1e-6, binding.LA_BF16)
    st = lib.lin_attn_prefill_noalloc(ctypes.byref(desc), fake, fake, fake, None, None, None, None, fake, None, None,
                                      None)
    assert st == binding.LA_ERR_WORKSPACE
    desc = binding.prefill_desc(1, 2, 4096, 128, 128, 128, 48, PSI_IDENTITY, 0, 1e-6, binding.LA_BF16)
    st = lib.lin_attn_prefill_noalloc(ctypes.byref(desc), fake, fake, fake, None, None, None, None, fake, None, None,
                                      None)
    assert st == binding.LA_ERR_UNSUPPORTED  # validation as lin_attn_prefill's
