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
  cpu_baseline  the fp64 oracle timed on this host's cores on a bounded sample.
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
                  out_dtype: torch.dtype = torch.float32):
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for row in evs:  # torch creates the HIP event on first record; the library re-records it
        for e in row:
            e.record()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        binding.lin_attn_prefill(inp["q"], inp["k"], inp["v"], events=evs[s], **kw)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    phases = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])] for e in evs])
    ms = total_ms / steps
    units = w.token_heads
    res = {
        "ms_per_step": ms,
        "token_heads_per_s": units / (ms * 1e-3),
        "phase_ms": {"summary": float(phases[:, 0].mean()), "scan": float(phases[:, 1].mean()),
                     "output": float(phases[:, 2].mean())},
        "units": units,
    }
    del inp, o, ws
    torch.cuda.empty_cache()
    return res


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
                                binding.LA_BF16, binding.LA_F32)
    ws = torch.empty(binding.backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    grads = [torch.empty((w.B, w.H, w.T, d), dtype=torch.float32, device="cuda") for d in (w.d_k, w.d_k, w.d_v)]
    kw = dict(psi=w.psi, chunk=w.chunk, normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g),
              dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
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


def bench_decode(w: workloads.DecodeWorkload, steps: int, warmup: int, replicas: int = 1):
    """steps consecutive decode launches, each on its own pre-generated token; state from a GPU prefill
    of the seeded prefix (the state only sets realistic magnitudes here; parity is tested elsewhere).
    replicas > 1 rotates the steps over that many copies of the state, so that consecutive steps do
    not find the (129 MiB) state in the 256 MB Infinity Cache: the HBM-bound rate."""
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
                                     normalize=w.normalize, eps=w.eps, gamma=gam, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_step_bytes = N * H * (2 * (d * d * 4 + d * 4) + 3 * d * 2 + d * 4)
    step_us = ms * 1e3 / steps
    del Ss, Zs, S0, Z0, toks
    torch.cuda.empty_cache()
    return {"steps_per_s": steps / (ms * 1e-3), "us_per_step": step_us, "bytes_per_step": per_step_bytes,
            "achieved_GBs": per_step_bytes / (step_us * 1e-6) / 1e9,
            "frac_of_hbm_peak": per_step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def copy_probe(mib: int):
    """One plain device-to-device copy of mib MiB: the reference kernel for scaling the HBM byte
    counters (FETCH_SIZE, WRITE_SIZE) of a counter run to bytes."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.neg(a, out=b)  # one elementwise kernel, the only negation in the run: reads mib MiB, writes mib MiB
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def cpu_baseline(w: workloads.Workload, budget_s: float):
    """The fp64 oracle on this host's cores over whole heads of the same workload, until budget_s."""
    import oracle
    # the host's CPU share: the affinity set, capped by OMP_NUM_THREADS when the environment sets it
    nthreads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        nthreads = max(1, min(nthreads, int(os.environ["OMP_NUM_THREADS"])))
    log(f"cpu baseline: fp64 oracle on {nthreads} threads, budget ~{budget_s:.0f}s")
    inp = inputs.make_prefill_inputs(w, device="cuda")
    gam = inp["gamma"]
    q = inp["q"].reshape(w.B * w.H, w.T, w.d_k)
    k = inp["k"].reshape(w.B * w.H, w.T, w.d_k)
    v = inp["v"].reshape(w.B * w.H, w.T, w.d_v)
    done_heads, elapsed = 0, 0.0
    batch = max(1, min(nthreads, 16))
    heads = list(range(w.B * w.H))
    while done_heads < len(heads) and elapsed < budget_s:
        sel = heads[done_heads:done_heads + batch]
        qs, ks, vs = q[sel].cpu(), k[sel].cpu(), v[sel].cpu()
        g = None if gam is None else [float(gam[b % w.H]) for b in sel]
        t = time.perf_counter()
        oracle.prefill(qs, ks, vs, w.psi, gamma=g, normalize=w.normalize, eps=float(np.float32(w.eps)),
                       nthreads=nthreads)
        elapsed += time.perf_counter() - t
        done_heads += len(sel)
    del inp, q, k, v
    torch.cuda.empty_cache()
    units = done_heads * w.T
    return {"value": units / elapsed, "unit": "token*heads/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{done_heads} of {w.B * w.H} heads x all {w.T} tokens of {w.name} (fp64 recurrence, "
                      f"OpenMP over heads, {elapsed:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only (no 8k elu+1, PRF, layout, bf16-output, gated, backward and packed-batch lines)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run one plain copy of MIB MiB (counter calibration)")
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

    w = workloads.RETNET_128K
    pre = bench_prefill(w, args.steps, args.warmup)
    out_ms = pre["phase_ms"]["output"]
    achieved = BYTES_PER_TOKEN_HEAD * pre["units"] / (out_ms * 1e-3) / 1e9
    traffic = traffic_from_profiles("k_output_retnet_128k")
    roofline = {"kernel": "k_output_sh<64,128>", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "whole_call_frac": round(BYTES_PER_TOKEN_HEAD * pre["units"] / (pre["ms_per_step"] * 1e-3) / 1e9
                                         / HBM_PEAK_GBS, 4)}
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
        "mfma_counters": {"output": mfma_from_profiles("k_output_retnet_128k"),
                          "summary": mfma_from_profiles("k_summary_retnet_128k")},
    }
    if not args.no_extra:
        prf_qs = workloads.PRF_4K.with_(name="prf256_4k_qshift", psi=workloads.PSI_PRF_QSHIFT)
        for key, wx, tag in (("prefill_8k", workloads.PREFILL_8K, "elu1_8k"),
                             ("prefill_prf_4k", workloads.PRF_4K, "prf256_4k"),
                             ("prefill_prf_4k_qshift", prf_qs, "prf256_4k_qshift")):
            px = bench_prefill(wx, args.steps, args.warmup)
            ax = BYTES_PER_TOKEN_HEAD * px["units"] / (px["ms_per_step"] * 1e-3) / 1e9
            line[key] = {"workload": wx.name, "token_heads_per_s": round(px["token_heads_per_s"], 1),
                         "ms_per_step": round(px["ms_per_step"], 4),
                         "phase_ms": {k: round(v, 4) for k, v in px["phase_ms"].items()},
                         "whole_call_roofline": {"bound": "hbm", "achieved": round(ax, 1), "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": round(ax / HBM_PEAK_GBS, 4)},
                         "mfma_counters": {"output": mfma_from_profiles(f"k_output_{tag}"),
                                           "summary": mfma_from_profiles(f"k_summary_{tag}")}}
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
        # backward: compulsory bytes per token-head (q, k, v bf16 and dout fp32 read; dq, dk, dv fp32 written)
        bwd_bytes = 3 * 128 * 2 + 128 * 4 + 3 * 128 * 4
        for key, bw in (("backward_8k", workloads.PREFILL_8K), ("backward_128k", workloads.RETNET_128K)):
            pb = bench_backward(bw, args.steps, args.warmup)
            ab = bwd_bytes * pb["units"] / (pb["ms_per_step"] * 1e-3) / 1e9
            line[key] = {"workload": bw.name, "token_heads_per_s": round(pb["token_heads_per_s"], 1),
                         "ms_per_step": round(pb["ms_per_step"], 4),
                         "whole_call_roofline": {"bound": "hbm", "achieved": round(ab, 1), "peak": HBM_PEAK_GBS,
                                                 "unit": "GB/s", "frac": round(ab / HBM_PEAK_GBS, 4),
                                                 "bytes_per_token_head": bwd_bytes}}
        vw = workloads.VARLEN_32
        pv = bench_varlen(vw, args.steps, args.warmup)
        av = BYTES_PER_TOKEN_HEAD * pv["units"] / (pv["ms_per_step"] * 1e-3) / 1e9
        line["prefill_varlen"] = {"workload": vw.name, "sequences": pv["lengths"], "H": vw.H, "chunk": vw.chunk,
                                  "token_heads_per_s": round(pv["token_heads_per_s"], 1),
                                  "ms_per_step": round(pv["ms_per_step"], 4),
                                  "whole_call_roofline": {"bound": "hbm", "achieved": round(av, 1),
                                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                          "frac": round(av / HBM_PEAK_GBS, 4)}}
    if not args.no_decode:
        dw = workloads.DECODE_32x64
        for key, reps, note in (("decode", 1, "as configured: the 129 MiB state is re-read every step and can "
                                 "be served partly from the 256 MB Infinity Cache (effective rate)"),
                                ("decode_cold", 4, "steps rotate over 4 state copies (516 MiB), so the state "
                                 "comes from HBM (HBM-bound rate)")):
            dec = bench_decode(dw, args.decode_steps, warmup=8, replicas=reps)
            line[key] = {"workload": dw.name, "steps": args.decode_steps,
                         "steps_per_s": round(dec["steps_per_s"], 1), "us_per_step": round(dec["us_per_step"], 3),
                         "roofline": {"bound": "hbm", "achieved": round(dec["achieved_GBs"], 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(dec["frac_of_hbm_peak"], 4),
                                      "traffic": traffic_from_profiles("k_decode_32x64") if reps == 1 else None},
                         "note": note}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
