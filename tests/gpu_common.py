"""Shared helpers for the GPU parity tests (comparison metrics and tolerances)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# Tolerances against the fp64 oracle: bf16 inputs with fp32 accumulation, and fp32 inputs.
BF16_REL_L2 = 2e-3
BF16_MAX_ABS = 1e-2
F32_REL_L2 = 1e-5


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU output"
    err = got - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.abs(err).max()) if err.size else 0.0


def assert_close(got, ref, dtype: str, label: str = ""):
    rel, mx = metrics(got, ref)
    print(f"[parity] {label} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    if dtype == "bf16":
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS, f"{label}: rel_l2={rel:.3e} max_abs={mx:.3e}"
    else:
        assert rel <= F32_REL_L2, f"{label}: rel_l2={rel:.3e}"
    return rel, mx


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def oracle_blocks(w, inp, heads=None, S0=None, Z0=None, want_state=False, nthreads: int = 0):
    """Oracle prefill outputs for the (b, h) blocks listed in heads (default all) of a workload's
    inputs (inputs.make_prefill_inputs, on any device), as fp64 [nblk, T, d_v]."""
    import oracle
    q, k, v = inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu()
    BH = w.B * w.H
    q, k, v = q.reshape(BH, w.T, -1), k.reshape(BH, w.T, -1), v.reshape(BH, w.T, -1)
    idx = list(range(BH)) if heads is None else list(heads)
    qs, ks, vs = q[idx].contiguous(), k[idx].contiguous(), v[idx].contiguous()
    g = inp["gamma"]
    gam = None if g is None else [float(g[b % w.H]) for b in idx]
    prf = inp.get("prf_w")
    return oracle.prefill(qs, ks, vs, w.psi, n_psi=w.n_psi, prf_w=None if prf is None else prf.cpu(),
                          w_head=[b % w.H for b in idx] if prf is not None else None, gamma=gam,
                          normalize=w.normalize, eps=float(np.float32(w.eps)), S0=S0, Z0=Z0,
                          want_state=want_state, nthreads=nthreads)


def compare_all_blocks(w, o, inp, label: str, group: int = 16):
    """Every output of a prefill workload against the oracle, streamed over groups of (b, h)
    blocks so that the fp64 reference of a large call never exists whole. Asserts the tolerance
    on the whole output (rel-L2 over all of it, max-abs over every element) and on each block's
    own rel-L2. Returns (rel_l2, max_abs, worst_block_rel_l2)."""
    BH = w.B * w.H
    o = o.reshape(BH, w.T, w.d_v)
    err2 = ref2 = 0.0
    mx = worst = 0.0
    for s in range(0, BH, group):
        idx = list(range(s, min(BH, s + group)))
        got = o[s:s + len(idx)].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), f"{label}: non-finite GPU outputs in blocks {idx[0]}..{idx[-1]}"
        ref = oracle_blocks(w, inp, heads=idx)
        err = got - ref
        e2 = (err * err).sum(axis=(1, 2))
        r2 = (ref * ref).sum(axis=(1, 2))
        worst = max(worst, float(np.sqrt(e2 / np.maximum(r2, 1e-300)).max()))
        err2 += float(e2.sum())
        ref2 += float(r2.sum())
        mx = max(mx, float(np.abs(err).max()))
        del got, ref, err
    rel = float(np.sqrt(err2 / max(ref2, 1e-300)))
    print(f"[parity] {label} all {BH} blocks: rel_l2={rel:.3e} max_abs={mx:.3e} worst block rel_l2={worst:.3e}",
          flush=True)
    if w.dtype == "bf16":
        assert rel <= BF16_REL_L2 and mx <= BF16_MAX_ABS and worst <= BF16_REL_L2, (label, rel, mx, worst)
    else:
        assert rel <= F32_REL_L2 and worst <= F32_REL_L2, (label, rel, worst)
    return rel, mx, worst
