#!/usr/bin/env python3
"""Benchmark of chunkwise causal linear attention on one MI355X.

Headline (the JSON line's `value`): prefill throughput, token*heads per second, on
the 128k-context decayed-retention workload -- B=1, H=64, T=131035 (ragged: the
last chunk has 91 tokens), d=128, C=128, identity feature map, per-head
gamma_h = 1 - 2^(-5 - 5h/63), no denominator, bf16 inputs, fp32 state and output.
One step = one lin_attn_prefill call over that whole batch (segment summaries,
segment scan, output pass), inputs resident in HBM before timing starts.

Also reported on the same line:
  roofline      the output kernel (the dominant one), algorithmic bytes / its
                average duration from HIP events over the timed region;
  decode        steps/s of lin_attn_decode_step on 32 streams x 64 heads
                (d=128, elu+1, gamma 0.999, state from a 4096-token prefix);
  cpu_baseline  the fp64 oracle timed on this host's cores (every block of the
                timed call), beside each configuration's own rate;
  parity        the timed outputs of every configuration against that oracle
                (rel-L2 and max-abs over every output; decode: all 256 steps).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from chunked_causal_linear_k1_amd import binding, inputs, workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 4   # q, k, v read once (bf16) + o written once (fp32), d = 128
PROFILE_DIR = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def traffic_from_profiles(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary (profiles/traffic.json,
    written by chunked_causal_linear_k1_amd.pmc_traffic), or None when it is absent or was taken
    on kernel sources other than the current ones."""
    from chunked_causal_linear_k1_amd import pmc_traffic
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != pmc_traffic.source_hash() or kernel_key not in rec:
        return None
    return rec[kernel_key]["bytes"]


def mfma_from_profiles(kernel_key: str):
    """rocprofv3 MFMA figures for one launch of a prefill kernel (profiles/mfma.json, written by
    chunked_causal_linear_k1_amd.pmc_mfma): busy percentage and executed bf16 MFMA flops, or None
    when absent or taken on kernel sources other than the current ones."""
    from chunked_causal_linear_k1_amd import pmc_traffic
    path = os.path.join(PROFILE_DIR, "mfma.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != pmc_traffic.source_hash() or kernel_key not in rec:
        return None
    r = rec[kernel_key]
    return {"kernel": kernel_key, "mfma_busy_pct": r["mfma_busy_pct"], "mfma_bf16_flops": r["mfma_bf16_flops"]}


def bench_prefill(w: workloads.Workload, steps: int, warmup: int, layout: str = "bhtd",
                  out_dtype: torch.dtype = torch.float32, keep: bool = False):
    """Event-timed lin_attn_prefill calls. keep: also return the inputs and the output of the
    last timed call (res["inp"], res["o"]) for the oracle comparison."""
    log(f"prefill {w.name} ({layout}, {out_dtype}): generating inputs on the GPU")
    inp = inputs.make_prefill_inputs(w, device="cuda")
    if layout == "bthd":  # the same tokens in [B, T, H, d]
        for key in ("q", "k", "v"):
            inp[key] = inp[key].transpose(1, 2).contiguous()
    g = inp["gamma"]
    gam = None if g is None else list(g)
    shape = (w.B, w.H, w.T, w.d_v) if layout == "bhtd" else (w.B, w.T, w.H, w.d_v)
    o = torch.empty(shape, dtype=out_dtype, device="cuda")
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_BF16, binding.LA_BF16 if out_dtype == torch.bfloat16 else binding.LA_F32,
                                binding.LA_LAYOUT_BHTD if layout == "bhtd" else binding.LA_LAYOUT_BTHD)
    ws = torch.empty(max(binding.workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=gam, prf_w=inp["prf_w"], o=o,
              workspace=ws, layout=layout)
    for _ in range(warmup):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], **kw)
    torch.cuda.synchronize()
    # whole calls as a caller makes them (no events inside the call)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    # then the same calls again with events between the three launches, for the phase split
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for row in evs:  # torch creates the HIP event on first record; the library re-records it
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for s in range(steps):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], events=evs[s], **kw)
    torch.cuda.synchronize()
    phases = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    units = w.token_heads
    res = {
        "ms_per_step": ms,
        "token_heads_per_s": units / (ms * 1e-3),
        "phase_ms": {"summary": float(phases[:, 0].mean()), "scan": float(phases[:, 1].mean()),
                     "output": float(phases[:, 2].mean())},
        "units": units,
    }
    if keep:
        res["inp"], res["o"] = inp, o
    del inp, o, ws
    torch.cuda.empty_cache()
    return res


def bench_tiny(w: workloads.Workload, calls: int, warmup: int):
    """The tiny fp32 workload: microseconds per lin_attn_prefill call (launch-latency bound),
    from events around `calls` back-to-back calls; keeps the inputs and the last output."""
    log(f"prefill {w.name}: generating inputs on the GPU")
    inp = inputs.make_prefill_inputs(w, device="cuda")
    o = torch.empty((w.B, w.H, w.T, w.d_v), dtype=torch.float32, device="cuda")
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_F32)
    ws = torch.empty(max(binding.workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, o=o, workspace=ws)
    for _ in range(warmup):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], **kw)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(calls):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], **kw)
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / calls
    return {"us_per_call": us, "token_heads_per_s": w.token_heads / (us * 1e-6), "units": w.token_heads,
            "inp": inp, "o": o}


def bench_gated(w: workloads.Workload, steps: int, warmup: int):
    """Whole lin_attn_prefill_gated calls (fp32 vector-ALU path), event-timed on the current stream."""
    log(f"prefill {w.name}: generating inputs and log gates on the GPU")
    inp = inputs.make_prefill_inputs(w, device="cuda")
    lg = inputs.make_log_gates((w.B, w.H, w.T, w.d_k), w.seed + 2, w.extra["gate_temp"], device="cuda")
    o = torch.empty((w.B, w.H, w.T, w.d_v), dtype=torch.float32, device="cuda")
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_BF16)
    ws = torch.empty(max(binding.gated_workspace_size(desc), 16), dtype=torch.uint8, device="cuda")
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, o=o, workspace=ws)
    for _ in range(warmup):
        binding.lin_attn_prefill_gated(inp["q"], inp["k"], inp["v"], lg, **kw)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        binding.lin_attn_prefill_gated(inp["q"], inp["k"], inp["v"], lg, **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    res = {"ms_per_step": ms, "token_heads_per_s": w.token_heads / (ms * 1e-3), "units": w.token_heads}
    del inp, lg, o, ws
    torch.cuda.empty_cache()
    return res


def bench_backward(w: workloads.Workload, steps: int, warmup: int):
    """Whole lin_attn_prefill_backward calls (forward summaries, scan, query sweep, reverse scan,
    state sweep) for an upstream gradient of o's shape, event-timed on the current stream."""
    log(f"backward {w.name}: generating inputs and the upstream gradient on the GPU")
    inp = inputs.make_prefill_inputs(w, device="cuda")
    dout = inputs.make_upstream_grad((w.B, w.H, w.T, w.d_v), w.seed + 11, device="cuda")
    g = inp["gamma"]
    desc = binding.prefill_desc(w.B, w.H, w.T, w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_F32 if w.dtype == "f32" else binding.LA_BF16, binding.LA_F32)
    ws = torch.empty(binding.backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    grads = [torch.empty((w.B, w.H, w.T, d), dtype=torch.float32, device="cuda") for d in (w.d_k, w.d_k, w.d_v)]
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g),
              prf_w=inp["prf_w"], dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
    for _ in range(warmup):
        binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        binding.lin_attn_prefill_backward(inp["q"], inp["k"], inp["v"], dout, **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    res = {"ms_per_step": ms, "token_heads_per_s": w.token_heads / (ms * 1e-3), "units": w.token_heads}
    del inp, dout, ws, grads
    torch.cuda.empty_cache()
    return res


def bench_varlen(w: workloads.VarlenWorkload, steps: int, warmup: int):
    """Whole lin_attn_prefill_varlen calls on a packed batch, event-timed on the current stream."""
    log(f"prefill {w.name}: generating packed inputs on the GPU")
    inp = inputs.make_varlen_inputs(w, device="cuda")
    g = inp["gamma"]
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g))
    o = torch.empty((inp["q"].shape[0], w.H, w.d_v), dtype=torch.float32, device="cuda")
    desc = binding.prefill_desc(w.N, w.H, inp["max_len"], w.d_k, w.d_v, w.n_psi, w.chunk, w.psi, w.normalize, w.eps,
                                binding.LA_BF16, binding.LA_F32, binding.LA_LAYOUT_BTHD)
    ws = torch.empty(max(binding.varlen_workspace_size(desc, inp["q"].shape[0]), 16), dtype=torch.uint8,
                     device="cuda")
    args = (inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["max_len"])
    for _ in range(warmup):
        binding.lin_attn_prefill_varlen(*args, o=o, workspace=ws, **kw)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        binding.lin_attn_prefill_varlen(*args, o=o, workspace=ws, **kw)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    units = sum(inp["lengths"]) * w.H
    res = {"ms_per_step": ms, "token_heads_per_s": units / (ms * 1e-3), "units": units,
           "lengths": {"n": w.N, "min": min(inp["lengths"]), "max": inp["max_len"], "total": sum(inp["lengths"])}}
    del inp, o, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(w: workloads.DecodeWorkload, steps: int, warmup: int, replicas: int = 1, keep: bool = False):
    """steps consecutive decode launches, each on its own pre-generated token; state from a GPU prefill
    of the seeded prefix (the state only sets realistic magnitudes here; parity is tested elsewhere).
    replicas > 1 rotates the steps over that many copies of the state, so that consecutive steps do
    not find the (129 MiB) state in the 256 MB Infinity Cache: the HBM-bound rate.
    keep (replicas == 1): every step writes its own output row, and the starting state, the
    step inputs, the outputs and the final state are returned for the oracle comparison."""
    log(f"decode {w.name}: building the state from a {w.prefix_len}-token prefix")
    prefix = inputs.make_decode_prefix(w, device="cuda")
    N, H, d = w.N, w.H, w.d_k
    S = torch.empty((N, H, d, d), dtype=torch.float32, device="cuda")
    Z = torch.empty((N, H, d), dtype=torch.float32, device="cuda")
    gam = [w.gamma] * H
    qp = torch.zeros_like(prefix["k"])
    binding.lin_attn_prefill(qp, prefix["k"], prefix["v"], psi=w.psi, chunk=64, normalize=w.normalize, eps=w.eps,
                             gamma=gam, final_S=S, final_Z=Z)
    del qp, prefix
    S0, Z0 = S.clone(), Z.clone()
    Ss = [S] + [S0.clone() for _ in range(replicas - 1)]
    Zs = [Z] + [Z0.clone() for _ in range(replicas - 1)]
    toks = inputs.make_decode_steps(w, steps=max(steps, warmup), device="cuda")
    o = torch.empty((N, H, d), dtype=torch.float32, device="cuda")
    o_all = torch.empty((steps, N, H, d), dtype=torch.float32, device="cuda") if keep else None
    q, k, v = toks["q"], toks["k"], toks["v"]
    for t in range(warmup):
        binding.lin_attn_decode_step(q[t], k[t], v[t], Ss[t % replicas], Zs[t % replicas], psi=w.psi,
                                     normalize=w.normalize, eps=w.eps, gamma=gam, o=o)
    for r in range(replicas):
        Ss[r].copy_(S0)
        Zs[r].copy_(Z0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(steps):
        binding.lin_attn_decode_step(q[t], k[t], v[t], Ss[t % replicas], Zs[t % replicas], psi=w.psi,
                                     normalize=w.normalize, eps=w.eps, gamma=gam, o=o if o_all is None else o_all[t])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_step_bytes = N * H * (2 * (d * d * 4 + d * 4) + 3 * d * 2 + d * 4)
    step_us = ms * 1e3 / steps
    res = {"steps_per_s": steps / (ms * 1e-3), "us_per_step": step_us, "bytes_per_step": per_step_bytes,
           "achieved_GBs": per_step_bytes / (step_us * 1e-6) / 1e9,
           "frac_of_hbm_peak": per_step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    if keep:
        res["kept"] = {"S0": S0, "Z0": Z0, "q": q[:steps], "k": k[:steps], "v": v[:steps], "o": o_all,
                       "S": Ss[0], "Z": Zs[0]}
    del Ss, Zs, S0, Z0, toks
    torch.cuda.empty_cache()
    return res


def stream_ceiling(w: workloads.Workload, reps: int = 10):
    """Plain streaming kernels with the byte patterns of the two prefill passes at the
    workload's size (probe/stream_probe.hip): three bf16 reads and one fp32 write per element
    (the output pass), and two bf16 reads (the summary pass). Their rates are the practical
    ceiling the memory-bound passes are compared with on the same box."""
    import ctypes
    from chunked_causal_linear_k1_amd import build as hip_build
    lib = ctypes.CDLL(hip_build.PROBE_LIB)
    lib.ccl_stream_mix.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_size_t, ctypes.c_void_p]
    lib.ccl_stream_read2.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
    lib.ccl_stream_read2_parts.restype = ctypes.c_size_t
    n = w.B * w.H * w.T * w.d_v
    q, k, v = (torch.ones(n, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty(n, dtype=torch.float32, device="cuda")
    part = torch.empty(lib.ccl_stream_read2_parts(), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    calls = {"mix": lambda: lib.ccl_stream_mix(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), n, st),
             "read2": lambda: lib.ccl_stream_read2(k.data_ptr(), v.data_ptr(), part.data_ptr(), n, st)}
    out = {}
    for name, fn in calls.items():
        for _ in range(2):
            assert fn() == 0, name
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n * (10 if name == "mix" else 4)
        out[name] = {"ms": round(ms, 4), "bytes": nbytes, "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    assert float(o[0]) == 2.0 and float(part.double().sum()) == float(n), "stream probe results"
    del q, k, v, o, part
    torch.cuda.empty_cache()
    return out


def copy_probe(mib: int):
    """Plain device-to-device copies of mib MiB and then mib/4 MiB: the reference kernels for
    scaling the HBM byte counters (FETCH_SIZE, WRITE_SIZE) of a counter run to bytes (two sizes,
    so that the scale is shown not to depend on the size)."""
    for size in (mib, mib // 4):
        n = size * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)  # one elementwise kernel, the only negations in the run: reads size MiB, writes size MiB
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()


def host_threads() -> int:
    """The host's CPU share: the affinity set, capped by OMP_NUM_THREADS when the environment sets it."""
    n = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        n = max(1, min(n, int(os.environ["OMP_NUM_THREADS"])))
    return n


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _tol(dtype: str):
    return {"rel_l2": 2e-3, "max_abs": 1e-2} if dtype == "bf16" else {"rel_l2": 1e-5}


def _verdict(rel, mx, worst, dtype):
    t = _tol(dtype)
    ok = rel <= t["rel_l2"] and worst <= t["rel_l2"] and mx <= t.get("max_abs", float("inf"))
    return {"rel_l2": float(f"{rel:.3e}"), "max_abs": float(f"{mx:.3e}"), "worst_block_rel_l2": float(f"{worst:.3e}"),
            "tolerance": t, "pass": bool(ok)}


def oracle_prefill_leg(w: workloads.Workload, inp, o, budget_s: float = 1e9, group: int = 16):
    """The fp64 oracle over the (b, h) blocks of the call that was just timed, in groups of
    `group` blocks until every block is done (or budget_s of oracle time is spent): the
    oracle's rate on this host (the recurrence only, no generation or comparison) and the
    element-wise comparison of the timed GPU output with it."""
    import oracle
    nthreads = host_threads()
    BH = w.B * w.H
    q = inp["q"].reshape(BH, w.T, w.d_k)
    k = inp["k"].reshape(BH, w.T, w.d_k)
    v = inp["v"].reshape(BH, w.T, w.d_v)
    og = o.reshape(BH, w.T, w.d_v)
    gam = inp["gamma"]
    prf = None if inp.get("prf_w") is None else inp["prf_w"].cpu()
    err2 = ref2 = mx = worst = elapsed = 0.0
    done = 0
    while done < BH and elapsed < budget_s:
        sel = list(range(done, min(BH, done + group)))
        qs, ks, vs = q[sel].cpu(), k[sel].cpu(), v[sel].cpu()
        g = None if gam is None else [float(gam[b % w.H]) for b in sel]
        t = time.perf_counter()
        ref = oracle.prefill(qs, ks, vs, w.psi, n_psi=w.n_psi, prf_w=prf,
                             w_head=None if prf is None else [b % w.H for b in sel], gamma=g, normalize=w.normalize,
                             eps=float(np.float32(w.eps)), nthreads=nthreads)
        elapsed += time.perf_counter() - t
        got = og[sel[0]:sel[-1] + 1].cpu().numpy().astype(np.float64)
        err = got - ref
        e2, r2 = (err * err).sum(axis=(1, 2)), (ref * ref).sum(axis=(1, 2))
        worst = max(worst, float(np.sqrt(e2 / np.maximum(r2, 1e-300)).max()))
        err2, ref2 = err2 + float(e2.sum()), ref2 + float(r2.sum())
        mx = max(mx, float(np.abs(err).max()) if np.all(np.isfinite(got)) else float("inf"))
        done += len(sel)
        del ref, got, err
    rel = float(np.sqrt(err2 / max(ref2, 1e-300)))
    par = _verdict(rel, mx, worst, w.dtype)
    par["blocks"] = f"{done} of {BH} (batch, head) blocks, every token"
    units = done * w.T
    cpu = {"value": round(units / elapsed, 1), "unit": "token*heads/s", "cores": nthreads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{done} of {BH} (batch, head) blocks x all {w.T} tokens of {w.name} (fp64 token-by-token "
                     f"recurrence, OpenMP over blocks, {elapsed:.2f} s)"}
    log(f"oracle {w.name}: {done}/{BH} blocks in {elapsed:.1f}s, rel_l2={rel:.2e} max_abs={mx:.2e}")
    return par, cpu


def oracle_decode_leg(w: workloads.DecodeWorkload, kept):
    """The fp64 oracle carried over the same decode steps from the same fp32 starting state
    (the GPU prefill's state of the prefix): timed (steps/s on this host) and compared with
    every step's GPU output and the final state and normaliser."""
    import oracle
    nthreads = host_threads()
    NH = w.N * w.H
    S = kept["S0"].cpu().double().numpy().reshape(NH, w.n_psi, w.d_v).copy()
    Z = kept["Z0"].cpu().double().numpy().reshape(NH, w.n_psi).copy()
    og = kept["o"].cpu().numpy().reshape(-1, NH, w.d_v)
    qs, ks, vs = (kept[x].cpu().reshape(-1, NH, w.d_k) for x in ("q", "k", "v"))
    n = og.shape[0]
    gam = [float(np.float32(w.gamma))] * NH
    err2 = ref2 = mx = worst = elapsed = 0.0
    for t in range(n):
        t0 = time.perf_counter()
        ref = oracle.decode_step(qs[t], ks[t], vs[t], S, Z, w.psi, gamma=gam, normalize=w.normalize,
                                 eps=float(np.float32(w.eps)), nthreads=nthreads)
        elapsed += time.perf_counter() - t0
        err = og[t].astype(np.float64) - ref
        e2, r2 = float((err * err).sum()), float((ref * ref).sum())
        worst = max(worst, np.sqrt(e2 / max(r2, 1e-300)))
        err2, ref2 = err2 + e2, ref2 + r2
        mx = max(mx, float(np.abs(err).max()))
    rel = float(np.sqrt(err2 / max(ref2, 1e-300)))
    par = _verdict(rel, mx, worst, "bf16")
    par["worst_step_rel_l2"] = par.pop("worst_block_rel_l2")
    par["steps"] = f"all {n} steps x {NH} (stream, head) states"
    gS = kept["S"].cpu().double().numpy().reshape(NH, w.n_psi, w.d_v)
    gZ = kept["Z"].cpu().double().numpy().reshape(NH, w.n_psi)
    par["final_S_rel_l2"] = float(f"{np.linalg.norm(gS - S) / np.linalg.norm(S):.3e}")
    par["final_Z_rel_l2"] = float(f"{np.linalg.norm(gZ - Z) / np.linalg.norm(Z):.3e}")
    par["pass"] = bool(par["pass"] and par["final_S_rel_l2"] <= 2e-3 and par["final_Z_rel_l2"] <= 2e-3)
    cpu = {"value": round(n / elapsed, 2), "unit": "steps/s", "cores": nthreads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"all {n} steps of {w.name} ({NH} states each, fp64, OpenMP over states, {elapsed:.2f} s)"}
    log(f"oracle {w.name}: {n} steps in {elapsed:.1f}s, rel_l2={rel:.2e} max_abs={mx:.2e}")
    return par, cpu


def _rate_vs_target(rate, target):
    return {"value": round(rate, 1), "target": target, "frac_of_target": round(rate / target, 4), "met": rate >= target}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle legs (timing of the fp64 oracle and parity of the timed outputs)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only (no 8k elu+1, PRF, layout, bf16-output, gated, backward and packed-batch lines)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run plain copies of MIB and MIB/4 MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              "(multi-GPU sequence/head sharding is described in the design notes, not built)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    binding.load()
    if args.copy_probe:
        copy_probe(args.copy_probe)
    oracle_legs = not args.no_cpu_baseline
    kept = {}  # workload name -> (workload, inputs, output) of the last timed call

    w = workloads.RETNET_128K
    pre = bench_prefill(w, args.steps, args.warmup, keep=oracle_legs)
    if oracle_legs:
        kept["headline"] = (w, pre.pop("inp"), pre.pop("o"))
    out_ms = pre["phase_ms"]["output"]
    achieved = BYTES_PER_TOKEN_HEAD * pre["units"] / (out_ms * 1e-3) / 1e9
    whole = BYTES_PER_TOKEN_HEAD * pre["units"] / (pre["ms_per_step"] * 1e-3) / 1e9
    traffic = traffic_from_profiles("k_output_retnet_128k")
    from chunked_causal_linear_k1_amd import pmc_traffic
    src = f"profiles/traffic.json (rocprofv3 FETCH_SIZE/WRITE_SIZE runs) at kernel-source hash {pmc_traffic.source_hash()}"
    roofline = {"kernel": "k_output_sh<64,128> (the output pass, the call's dominant kernel)", "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_source": src if traffic is not None else "no counter run on the current kernel sources",
                "bytes_per_unit": BYTES_PER_TOKEN_HEAD, "units_per_launch": pre["units"]}
    line = {
        "metric": "prefill tokens*heads/s at 128k (decayed retention, ragged T)",
        "value": round(pre["token_heads_per_s"], 1),
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk,
                   "psi": "identity", "decay": "gamma_h = 1 - 2^(-5-5h/63)", "normalize": 0,
                   "state": "fp32", "output": "fp32"},
        "phase_ms": {k: round(v, 4) for k, v in pre["phase_ms"].items()},
        "roofline": roofline,
        # the prefill target (half the HBM roofline) applies to the whole call, not to one kernel
        "whole_call_roofline": {"bound": "hbm", "achieved": round(whole, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(whole / HBM_PEAK_GBS, 4), "target_frac": 0.5,
                                "met": whole / HBM_PEAK_GBS >= 0.5},
        "mfma_counters": {"output": mfma_from_profiles("k_output_retnet_128k"),
                          "summary": mfma_from_profiles("k_summary_retnet_128k"),
                          "source": "profiles/mfma.json (rocprofv3 MfmaUtil and SQ_INSTS_VALU_MFMA_MOPS_BF16 runs) at "
                                    f"kernel-source hash {pmc_traffic.source_hash()}; null when taken on other sources"},
    }
    targets = {"prefill_128k": _rate_vs_target(pre["token_heads_per_s"], 3.125e9)}
    sc = stream_ceiling(w)
    sum_bytes = 4 * w.d_v * pre["units"]  # k and v read once (the records are 1.3% more)
    sum_gbs = sum_bytes / (pre["phase_ms"]["summary"] * 1e-3) / 1e9
    line["stream_ceiling"] = {
        "note": "plain streaming kernels with each pass's byte pattern at this size, timed in this run",
        "output_pattern": sc["mix"], "summary_pattern": sc["read2"],
        "output_pass_of_stream": round(achieved / sc["mix"]["GBs"], 4),
        "summary_pass_of_stream": round(sum_gbs / sc["read2"]["GBs"], 4)}

    tw = workloads.TINY_F32
    pt = bench_tiny(tw, 200, 20)
    if oracle_legs:
        kept["tiny_f32"] = (tw, pt.pop("inp"), pt.pop("o"))
    else:
        pt.pop("inp"), pt.pop("o")
    line["tiny_f32"] = {"workload": tw.name, "us_per_call": round(pt["us_per_call"], 2),
                        "token_heads_per_s": round(pt["token_heads_per_s"], 1),
                        "note": "1 MiB of traffic per call: bound by launch latency, parity is its target"}
    if not args.no_extra:
        prf_qs = workloads.PRF_4K.with_(name="prf256_4k_qshift", psi=workloads.PSI_PRF_QSHIFT)
        for key, wx, tag in (("prefill_8k", workloads.PREFILL_8K, "elu1_8k"),
                             ("prefill_prf_4k", workloads.PRF_4K, "prf256_4k"),
                             ("prefill_prf_4k_qshift", prf_qs, "prf256_4k_qshift")):
            px = bench_prefill(wx, args.steps, args.warmup, keep=oracle_legs)
            if oracle_legs:
                kept[key] = (wx, px.pop("inp"), px.pop("o"))
            ax = BYTES_PER_TOKEN_HEAD * px["units"] / (px["ms_per_step"] * 1e-3) / 1e9
            line[key] = {"workload": wx.name, "token_heads_per_s": round(px["token_heads_per_s"], 1),
                         "ms_per_step": round(px["ms_per_step"], 4),
                         "phase_ms": {k: round(v, 4) for k, v in px["phase_ms"].items()},
                         "whole_call_roofline": {"bound": "hbm", "achieved": round(ax, 1), "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": round(ax / HBM_PEAK_GBS, 4)},
                         "mfma_counters": {"output": mfma_from_profiles(f"k_output_{tag}"),
                                           "summary": mfma_from_profiles(f"k_summary_{tag}")}}
            targets[key] = _rate_vs_target(px["token_heads_per_s"], 3.125e9)
            if wx.psi in (workloads.PSI_PRF, workloads.PSI_PRF_QSHIFT):
                # 286,720 algorithmic FLOP per token-head (features 4*256*128, local pass C*(256+128),
                # state and output 4*256*128); bf16 MFMA dense peak 2.5 PFLOP/s
                tf = 286720 * px["units"] / (px["ms_per_step"] * 1e-3) / 1e12
                line[key]["mfma_roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": 2500.0,
                                              "unit": "TFLOP/s", "frac": round(tf / 2500.0, 4)}
        # the 128k workload in the other token layout and with bf16 output (o = the fp32 result
        # rounded to nearest even: 768 + 256 algorithmic bytes per token-head)
        for key, layout, odt, bpt in (("prefill_128k_bthd", "bthd", torch.float32, BYTES_PER_TOKEN_HEAD),
                                      ("prefill_128k_bf16_out", "bhtd", torch.bfloat16, 3 * 128 * 2 + 128 * 2)):
            px = bench_prefill(w, args.steps, args.warmup, layout=layout, out_dtype=odt)
            ao = bpt * px["units"] / (px["phase_ms"]["output"] * 1e-3) / 1e9
            ax = bpt * px["units"] / (px["ms_per_step"] * 1e-3) / 1e9
            line[key] = {"workload": w.name, "layout": layout, "output": str(odt).replace("torch.", ""),
                         "token_heads_per_s": round(px["token_heads_per_s"], 1),
                         "ms_per_step": round(px["ms_per_step"], 4),
                         "phase_ms": {k: round(v, 4) for k, v in px["phase_ms"].items()},
                         "roofline": {"kernel": "output pass", "bound": "hbm", "achieved": round(ao, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ao / HBM_PEAK_GBS, 4),
                                      "bytes_per_token_head": bpt},
                         "whole_call_roofline": {"bound": "hbm", "achieved": round(ax, 1), "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": round(ax / HBM_PEAK_GBS, 4)}}
        gw = workloads.GATED_8K
        pg = bench_gated(gw, args.steps, args.warmup)
        # compulsory bytes per token-head: q, k, v bf16, the fp32 log gates, o fp32. The state terms
        # run on MFMA and the scores on the vector ALUs; at C*n + C*d_v + 4*n*d_v FLOP per
        # token-head (~41 FLOP/B) the path sits below the MFMA ridge, so HBM is its roofline
        gbytes = 3 * 128 * 2 + 128 * 4 + 128 * 4
        flop = gw.chunk * gw.n_psi + gw.chunk * gw.d_v + 4 * gw.n_psi * gw.d_v
        gb = gbytes * pg["units"] / (pg["ms_per_step"] * 1e-3) / 1e9
        tf = flop * pg["units"] / (pg["ms_per_step"] * 1e-3) / 1e12
        line["prefill_gated_8k"] = {"workload": gw.name, "token_heads_per_s": round(pg["token_heads_per_s"], 1),
                                    "ms_per_step": round(pg["ms_per_step"], 4),
                                    "whole_call_roofline": {"bound": "hbm", "achieved": round(gb, 1),
                                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                            "frac": round(gb / HBM_PEAK_GBS, 4),
                                                            "bytes_per_token_head": gbytes},
                                    "algorithmic_tflops": round(tf, 1), "flop_per_token_head": flop}
        # backward: compulsory bytes per token-head (q, k, v and dout fp32 read; dq, dk, dv fp32 written)
        for key, bw in (("backward_8k", workloads.PREFILL_8K), ("backward_128k", workloads.RETNET_128K),
                        ("backward_prf_4k", workloads.PRF_4K), ("backward_tiny_f32", workloads.TINY_F32)):
            ib = 4 if bw.dtype == "f32" else 2
            bwd_bytes = 3 * bw.d_k * ib + bw.d_v * 4 + 3 * bw.d_k * 4
            pb = bench_backward(bw, args.steps, args.warmup)
            ab = bwd_bytes * pb["units"] / (pb["ms_per_step"] * 1e-3) / 1e9
            line[key] = {"workload": bw.name, "token_heads_per_s": round(pb["token_heads_per_s"], 1),
                         "ms_per_step": round(pb["ms_per_step"], 4),
                         "whole_call_roofline": {"bound": "hbm", "achieved": round(ab, 1), "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": round(ab / HBM_PEAK_GBS, 4),
                                                 "bytes_per_token_head": bwd_bytes}}
            if bw.dtype == "f32":  # the fp32 vector-ALU sweeps at the tiny fp32 shape: latency, not bandwidth
                line[key]["us_per_call"] = round(pb["ms_per_step"] * 1e3, 2)
                line[key]["note"] = "fp32 inputs (vector-ALU sweeps); bound by its chain of launches, like the forward"
        vw = workloads.VARLEN_32
        pv = bench_varlen(vw, args.steps, args.warmup)
        av = BYTES_PER_TOKEN_HEAD * pv["units"] / (pv["ms_per_step"] * 1e-3) / 1e9
        line["prefill_varlen"] = {"workload": vw.name, "sequences": pv["lengths"], "H": vw.H, "chunk": vw.chunk,
                                  "token_heads_per_s": round(pv["token_heads_per_s"], 1),
                                  "ms_per_step": round(pv["ms_per_step"], 4),
                                  "whole_call_roofline": {"bound": "hbm", "achieved": round(av, 1),
                                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                          "frac": round(av / HBM_PEAK_GBS, 4)}}
    dec_kept = None
    if not args.no_decode:
        dw = workloads.DECODE_32x64
        for key, reps, note in (("decode", 1, "as configured: the 129 MiB state is re-read every step and can "
                                 "be served partly from the 256 MB Infinity Cache (an effective, cache-assisted "
                                 "rate, not an HBM figure)"),
                                ("decode_cold", 4, "steps rotate over 4 state copies (516 MiB), so the state "
                                 "comes from HBM: the HBM-bound rate, scored against the 70%-of-HBM target")):
            dec = bench_decode(dw, args.decode_steps, warmup=8, replicas=reps, keep=oracle_legs and reps == 1)
            if "kept" in dec:
                dec_kept = dec.pop("kept")
            line[key] = {"workload": dw.name, "steps": args.decode_steps,
                         "steps_per_s": round(dec["steps_per_s"], 1), "us_per_step": round(dec["us_per_step"], 3),
                         "roofline": {"bound": "hbm", "achieved": round(dec["achieved_GBs"], 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(dec["frac_of_hbm_peak"], 4),
                                      "traffic": traffic_from_profiles("k_decode_32x64") if reps == 1 else None},
                         "note": note}
        targets["decode_cold"] = _rate_vs_target(line["decode_cold"]["steps_per_s"], 20500.0)
    line["targets"] = targets
    if oracle_legs:
        # the oracle on this host's cores beside each timed configuration: its rate, and the
        # comparison of the GPU output that was just timed (every block of every prefill config,
        # every decode step)
        parity = {}
        for key, (wx, inp, o) in kept.items():
            par, cpu = oracle_prefill_leg(wx, inp, o)
            parity[key] = par
            if key == "headline":
                line["cpu_baseline"] = cpu
            else:
                line[key]["cpu_baseline"] = cpu
            del inp, o
        kept.clear()
        torch.cuda.empty_cache()
        if dec_kept is not None:
            par, cpu = oracle_decode_leg(workloads.DECODE_32x64, dec_kept)
            parity["decode"] = par
            line["decode"]["cpu_baseline"] = cpu
        line["parity"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
