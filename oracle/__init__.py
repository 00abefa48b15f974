"""fp64 CPU oracle for chunkwise causal linear attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The product path (the HIP library and its binding)
never imports, links or calls it, and this package imports nothing from the
product package.

Contents
  * ``linattn_oracle.c`` -> ``liblinattn_oracle.so``: the token-by-token fp64
    recurrence (the definition; pinned by the tests listed in each function), and
    its adjoint for the backward pass (``prefill_backward``: a forward sweep for the
    query gradients and a reverse sweep over the adjoint state for the key and
    value gradients; pinned by finite differences of the forward oracle, autograd of
    the quadratic form and exact dyadic cases in tests/test_oracle_backward_pins.py).
  * ``brute.py``: the masked quadratic ("parallel") form, a second definition
    used to pin the recurrence on tiny inputs.
  * ``chunked.py``: an fp64 statement of the chunked method (chunk summaries,
    the monoid, exclusive scans in three orders) used to pin that chunking plus
    a scan reproduces the sequential result.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblinattn_oracle.so")
# A test that plants a mistake in a copy of the oracle points this at the copy.
_LIB_OVERRIDE = os.environ.get("LINATTN_ORACLE_LIB")

PSI_IDENTITY, PSI_ELU1, PSI_PRF, PSI_PRF_QSHIFT = 0, 1, 2, 3
BF16, F32 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        vp, dp, ip = ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)
        lib.oracle_prefill_f64.restype = ctypes.c_int
        lib.oracle_prefill_f64.argtypes = [ctypes.c_int] * 7 + [vp, vp, vp, vp, ip, dp, ctypes.c_int,
                                                                  ctypes.c_double, dp, dp, dp, dp, dp,
                                                                  ctypes.c_int]
        lib.oracle_decode_step_f64.restype = ctypes.c_int
        lib.oracle_decode_step_f64.argtypes = [ctypes.c_int] * 6 + [vp, vp, vp, vp, ip, dp, ctypes.c_int,
                                                                      ctypes.c_double, dp, dp, dp,
                                                                      ctypes.c_int]
        fp = ctypes.POINTER(ctypes.c_float)
        lib.oracle_prefill_gated_f64.restype = ctypes.c_int
        lib.oracle_prefill_gated_f64.argtypes = [ctypes.c_int] * 7 + [vp, vp, vp, vp, ip, fp, ctypes.c_int,
                                                                        ctypes.c_double, dp, dp, dp, dp, dp,
                                                                        ctypes.c_int]
        lib.oracle_decode_step_gated_f64.restype = ctypes.c_int
        lib.oracle_decode_step_gated_f64.argtypes = [ctypes.c_int] * 6 + [vp, vp, vp, vp, ip, fp, ctypes.c_int,
                                                                            ctypes.c_double, dp, dp, dp,
                                                                            ctypes.c_int]
        lib.oracle_prefill_backward_f64.restype = ctypes.c_int
        lib.oracle_prefill_backward_f64.argtypes = [ctypes.c_int] * 7 + [vp, vp, vp, vp, ip, dp, ctypes.c_int,
                                                                           ctypes.c_double, dp, dp, dp, dp, dp,
                                                                           dp, dp, dp, ctypes.c_int]
        lib.oracle_feature_f64.restype = None
        lib.oracle_feature_f64.argtypes = [ctypes.c_int] * 3 + [dp, dp, dp]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stored(x) -> tuple:
    """(contiguous numpy array of the stored bits, dtype code). Accepts torch CPU tensors or numpy."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError(f"unsupported stored dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"unsupported stored dtype {x.dtype}")


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def prefill(q, k, v, psi: int, n_psi: Optional[int] = None, prf_w=None, w_head=None, gamma=None,
            normalize: int = 1, eps: float = 1e-6, S0=None, Z0=None, want_state: bool = False,
            nthreads: int = 0, log_gate=None):
    """Oracle prefill for blocks [nblk, T, d] (leading dims are flattened into blocks).

    gamma: per-block decay values (anything array-like; each is used as given, in fp64) or None.
    w_head: per-block index into prf_w's first dim (or None -> 0). eps is used as given (fp64).
    Returns o [..., T, d_v] as float64 (or None if q is None), plus (S, Z) if want_state.
    """
    lib = _load()
    kk, dt = _stored(k)
    vv, dt2 = _stored(v)
    assert dt == dt2
    lead = kk.shape[:-2]
    T, d_k = kk.shape[-2], kk.shape[-1]
    d_v = vv.shape[-1]
    nblk = int(np.prod(lead)) if len(lead) else 1
    n_psi = d_k if n_psi is None else n_psi
    qq = None
    if q is not None:
        qq, dt3 = _stored(q)
        assert dt3 == dt and qq.shape == kk.shape
    ww = None
    if prf_w is not None:
        ww, dtw = _stored(prf_w)
        assert dtw == dt, "PRF bank must be stored like q/k/v"
    wh = None
    if w_head is not None:
        wh = np.ascontiguousarray(np.asarray(w_head, dtype=np.int32).reshape(nblk))
    g = None
    if gamma is not None:
        g = np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(nblk))
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64).reshape(nblk, n_psi, d_v))
    z0 = None if Z0 is None else np.ascontiguousarray(np.asarray(Z0, dtype=np.float64).reshape(nblk, n_psi))
    o = np.empty(lead + (T, d_v), dtype=np.float64) if qq is not None else None
    S = np.empty((nblk, n_psi, d_v), dtype=np.float64) if want_state else None
    Z = np.empty((nblk, n_psi), dtype=np.float64) if want_state else None
    if log_gate is not None:
        # per-token, per-state-row forget gates exp(log_gate) in place of gamma (fp32 values)
        lgt = _gate_f32(log_gate, (nblk, T, n_psi))
        rc = lib.oracle_prefill_gated_f64(
            nblk, T, d_k, d_v, n_psi, psi, dt,
            None if qq is None else qq.ctypes.data, kk.ctypes.data, vv.ctypes.data,
            None if ww is None else ww.ctypes.data,
            None if wh is None else wh.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            lgt.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(normalize), float(eps), _dptr(s0), _dptr(z0),
            _dptr(o), _dptr(S), _dptr(Z), int(nthreads))
    else:
        rc = lib.oracle_prefill_f64(
            nblk, T, d_k, d_v, n_psi, psi, dt,
            None if qq is None else qq.ctypes.data, kk.ctypes.data, vv.ctypes.data,
            None if ww is None else ww.ctypes.data,
            None if wh is None else wh.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            _dptr(g), int(normalize), float(eps), _dptr(s0), _dptr(z0), _dptr(o), _dptr(S), _dptr(Z),
            int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_prefill_f64 failed")
    if want_state:
        return o, S.reshape(lead + (n_psi, d_v)), Z.reshape(lead + (n_psi,))
    return o


def prefill_backward(q, k, v, dout, psi: int, n_psi: Optional[int] = None, prf_w=None, w_head=None,
                     gamma=None, normalize: int = 1, eps: float = 1e-6, S0=None, Z0=None, nthreads: int = 0):
    """Gradients of sum_t dout_t . o_t for the prefill of ``prefill`` (same arguments; dout is
    [..., T, d_v], any float type, used exactly in fp64). Returns fp64 (dq, dk, dv, dS0, dZ0)
    with the shapes of q, k, v and of the state [..., n_psi, d_v], [..., n_psi]."""
    lib = _load()
    qq, dt = _stored(q)
    kk, dt2 = _stored(k)
    vv, dt3 = _stored(v)
    assert dt == dt2 == dt3 and qq.shape == kk.shape
    lead = kk.shape[:-2]
    T, d_k = kk.shape[-2], kk.shape[-1]
    d_v = vv.shape[-1]
    nblk = int(np.prod(lead)) if len(lead) else 1
    n_psi = d_k if n_psi is None else n_psi
    ww = None
    if prf_w is not None:
        ww, dtw = _stored(prf_w)
        assert dtw == dt, "PRF bank must be stored like q/k/v"
    wh = None if w_head is None else np.ascontiguousarray(np.asarray(w_head, dtype=np.int32).reshape(nblk))
    g = None if gamma is None else np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(nblk))
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, dtype=np.float64).reshape(nblk, n_psi, d_v))
    z0 = None if Z0 is None else np.ascontiguousarray(np.asarray(Z0, dtype=np.float64).reshape(nblk, n_psi))
    do = np.ascontiguousarray(as_f64(dout).reshape(nblk, T, d_v))
    dq = np.empty(lead + (T, d_k), dtype=np.float64)
    dk = np.empty(lead + (T, d_k), dtype=np.float64)
    dv = np.empty(lead + (T, d_v), dtype=np.float64)
    dS0 = np.empty((nblk, n_psi, d_v), dtype=np.float64)
    dZ0 = np.empty((nblk, n_psi), dtype=np.float64)
    rc = lib.oracle_prefill_backward_f64(
        nblk, T, d_k, d_v, n_psi, psi, dt, qq.ctypes.data, kk.ctypes.data, vv.ctypes.data,
        None if ww is None else ww.ctypes.data,
        None if wh is None else wh.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        _dptr(g), int(normalize), float(eps), _dptr(s0), _dptr(z0), _dptr(do), _dptr(dq), _dptr(dk), _dptr(dv),
        _dptr(dS0), _dptr(dZ0), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_prefill_backward_f64 failed")
    return dq, dk, dv, dS0.reshape(lead + (n_psi, d_v)), dZ0.reshape(lead + (n_psi,))


def _gate_f32(log_gate, shape) -> np.ndarray:
    """log gates as a contiguous fp32 array of the given shape (fp32 values kept exactly)."""
    try:
        import torch
        if isinstance(log_gate, torch.Tensor):
            log_gate = log_gate.detach().cpu().float().numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(log_gate, dtype=np.float32))
    if a.size != int(np.prod(shape)):
        raise ValueError(f"log_gate has {a.size} values, expected {shape}")
    return a.reshape(shape)


def decode_step(q, k, v, S, Z, psi: int, prf_w=None, w_head=None, gamma=None, normalize: int = 1,
                eps: float = 1e-6, nthreads: int = 0, log_gate=None):
    """One in-place decode step on fp64 state S [nblk, n_psi, d_v], Z [nblk, n_psi]. Returns o (fp64)."""
    lib = _load()
    qq, dt = _stored(q)
    kk, _ = _stored(k)
    vv, _ = _stored(v)
    d_k, d_v = kk.shape[-1], vv.shape[-1]
    nblk = int(np.prod(kk.shape[:-1]))
    assert S.dtype == np.float64 and S.flags.c_contiguous
    n_psi = S.shape[-2]
    ww = None
    if prf_w is not None:
        ww, _ = _stored(prf_w)
    wh = None if w_head is None else np.ascontiguousarray(np.asarray(w_head, dtype=np.int32).reshape(nblk))
    g = None if gamma is None else np.ascontiguousarray(np.asarray(gamma, dtype=np.float64).reshape(nblk))
    if Z is not None:
        assert Z.dtype == np.float64 and Z.flags.c_contiguous
    o = np.empty(kk.shape[:-1] + (d_v,), dtype=np.float64)
    if log_gate is not None:
        lgt = _gate_f32(log_gate, (nblk, n_psi))
        rc = lib.oracle_decode_step_gated_f64(
            nblk, d_k, d_v, n_psi, psi, dt, qq.ctypes.data, kk.ctypes.data, vv.ctypes.data,
            None if ww is None else ww.ctypes.data,
            None if wh is None else wh.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            lgt.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), int(normalize), float(eps), _dptr(S), _dptr(Z),
            _dptr(o), int(nthreads))
    else:
        rc = lib.oracle_decode_step_f64(
            nblk, d_k, d_v, n_psi, psi, dt, qq.ctypes.data, kk.ctypes.data, vv.ctypes.data,
            None if ww is None else ww.ctypes.data,
            None if wh is None else wh.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
            _dptr(g), int(normalize), float(eps), _dptr(S), _dptr(Z), _dptr(o), int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_decode_step_f64 failed")
    return o


def feature(x: np.ndarray, psi: int, n_psi: Optional[int] = None, w: Optional[np.ndarray] = None) -> np.ndarray:
    """psi(x) for one fp64 vector x (and fp64 bank w [n_psi, d_k] for PRF)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    d_k = x.shape[0]
    n_psi = d_k if n_psi is None else n_psi
    wd = None if w is None else np.ascontiguousarray(w, dtype=np.float64)
    out = np.empty(n_psi, dtype=np.float64)
    lib.oracle_feature_f64(psi, d_k, n_psi, _dptr(x), _dptr(wd), _dptr(out))
    return out


def as_f64(x) -> np.ndarray:
    """Exact fp64 copy of a stored tensor (bf16 or fp32)."""
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)
