"""ctypes binding of liblinattn.so -- argument marshalling only.

Every function here turns torch tensors into the pointers and sizes the C ABI
(include/linattn.h) takes, calls it on torch's current HIP stream, and raises on
a non-OK status. All computation happens in the library's HIP kernels; there is
no fallback path. Device memory (outputs, workspace) comes from torch's caching
allocator.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

from . import workloads

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_ALIGN, LA_ERR_VALUE, LA_ERR_HIP = range(8)
LA_BF16, LA_F32 = 0, 1
LA_LAYOUT_BHTD, LA_LAYOUT_BTHD = 0, 1
MAX_DECAY_HEADS = 256

EXPORTED = ("lin_attn_prefill_workspace_size", "lin_attn_prefill", "lin_attn_prefill_profiled",
            "lin_attn_prefill_varlen", "lin_attn_prefill_varlen_workspace_size", "lin_attn_prefill_gated",
            "lin_attn_prefill_gated_workspace_size", "lin_attn_prefill_backward",
            "lin_attn_prefill_backward_workspace_size", "lin_attn_prefill_backward_varlen",
            "lin_attn_prefill_backward_varlen_workspace_size", "lin_attn_decode_step", "lin_attn_decode_step_gated",
            "lin_attn_status_string", "lin_attn_version", "lin_attn_prefill_noalloc", "lin_attn_scan_depth")
NOALLOC_SCRATCH_BYTES = 64 << 20  # LA_NOALLOC_SCRATCH_BYTES


class PrefillDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("n_psi", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("psi", ctypes.c_int32), ("normalize", ctypes.c_int32),
                ("eps", ctypes.c_float), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("H", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("n_psi", ctypes.c_int32), ("psi", ctypes.c_int32),
                ("normalize", ctypes.c_int32), ("eps", ctypes.c_float), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load liblinattn.so; raises if it has not been built (there is no other path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m chunked_causal_linear_k1_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        vp, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)
        lib.lin_attn_prefill_workspace_size.restype = ctypes.c_int
        lib.lin_attn_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.lin_attn_prefill.restype = ctypes.c_int
        lib.lin_attn_prefill.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, fp, vp, vp, vp, vp, vp, vp, vp,
                                         ctypes.c_size_t, vp]
        lib.lin_attn_prefill_profiled.restype = ctypes.c_int
        lib.lin_attn_prefill_profiled.argtypes = lib.lin_attn_prefill.argtypes + [ctypes.POINTER(ctypes.c_void_p)]
        lib.lin_attn_prefill_varlen.restype = ctypes.c_int
        lib.lin_attn_prefill_varlen_workspace_size.restype = ctypes.c_int
        lib.lin_attn_prefill_varlen_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_int32,
                                                               ctypes.POINTER(ctypes.c_size_t)]
        lib.lin_attn_prefill_varlen.argtypes = [ctypes.POINTER(PrefillDesc), vp, ctypes.c_int32, vp, vp, vp, fp, vp,
                                                vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.lin_attn_prefill_gated.restype = ctypes.c_int
        lib.lin_attn_prefill_gated.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               ctypes.c_size_t, vp]
        lib.lin_attn_prefill_gated_workspace_size.restype = ctypes.c_int
        lib.lin_attn_prefill_gated_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc),
                                                              ctypes.POINTER(ctypes.c_size_t)]
        lib.lin_attn_prefill_backward.restype = ctypes.c_int
        lib.lin_attn_prefill_backward.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, fp, vp, vp, vp, vp, vp,
                                                  vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        lib.lin_attn_prefill_backward_workspace_size.restype = ctypes.c_int
        lib.lin_attn_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc),
                                                                 ctypes.POINTER(ctypes.c_size_t)]
        lib.lin_attn_prefill_backward_varlen.restype = ctypes.c_int
        lib.lin_attn_prefill_backward_varlen.argtypes = [ctypes.POINTER(PrefillDesc), vp, ctypes.c_int32, vp, vp, vp,
                                                         fp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                         vp]
        lib.lin_attn_prefill_backward_varlen_workspace_size.restype = ctypes.c_int
        lib.lin_attn_prefill_backward_varlen_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_int32,
                                                                        ctypes.POINTER(ctypes.c_size_t)]
        lib.lin_attn_decode_step_gated.restype = ctypes.c_int
        lib.lin_attn_decode_step_gated.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.lin_attn_decode_step.restype = ctypes.c_int
        lib.lin_attn_decode_step.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, vp, fp, vp, vp, vp, vp, vp]
        lib.lin_attn_prefill_noalloc.restype = ctypes.c_int
        lib.lin_attn_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillDesc), vp, vp, vp, fp, vp, vp, vp, vp, vp, vp,
                                                 vp]
        lib.lin_attn_scan_depth.restype = ctypes.c_int
        lib.lin_attn_scan_depth.argtypes = [ctypes.c_int32, vp, vp, vp]
        lib.lin_attn_status_string.restype = ctypes.c_char_p
        lib.lin_attn_status_string.argtypes = [ctypes.c_int]
        lib.lin_attn_version.restype = ctypes.c_char_p
        lib.lin_attn_version.argtypes = []
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().lin_attn_status_string(int(status)).decode()


def version() -> str:
    return load().lin_attn_version().decode()


def scan_depth(n_seg: int, records: Optional[torch.Tensor] = None):
    """lin_attn_scan_depth: the segment scan over n_seg records of 20 floats (4 x 4 state, then
    4 normaliser entries; zeros unless given). Returns (rounds, prefixes): the dependent
    combine levels the kernel executed, and the exclusive prefixes it wrote [n_seg, 20]."""
    ws = (torch.zeros(max(1, n_seg) * 20, dtype=torch.float32, device="cuda") if records is None
          else records.to(device="cuda", dtype=torch.float32).contiguous().reshape(-1).clone())
    rounds = torch.zeros(1, dtype=torch.int32, device="cuda")
    st = load().lin_attn_scan_depth(int(n_seg), ws.data_ptr(), rounds.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise RuntimeError(f"lin_attn_scan_depth: {status_string(st)}")
    torch.cuda.synchronize()
    return int(rounds.item()), ws.reshape(-1, 20)[:n_seg]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gamma_array(gamma, H: int):
    if gamma is None:
        return None
    vals = [float(g) for g in gamma]
    if len(vals) != H:
        raise ValueError(f"gamma has {len(vals)} entries, expected H={H}")
    return (ctypes.c_float * H)(*vals)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def prefill_desc(B, H, T, d_k, d_v, n_psi, chunk, psi, normalize, eps, in_dtype, out_dtype=LA_F32,
                 layout=LA_LAYOUT_BHTD) -> PrefillDesc:
    return PrefillDesc(B, H, T, d_k, d_v, n_psi, chunk, psi, normalize, eps, in_dtype, out_dtype, layout)


def workspace_size(desc: PrefillDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load().lin_attn_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_workspace_size")
    return int(n.value)


def varlen_workspace_size(desc: PrefillDesc, total_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().lin_attn_prefill_varlen_workspace_size(ctypes.byref(desc), int(total_tokens), ctypes.byref(n))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_varlen_workspace_size")
    return int(n.value)


def lin_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, psi: int, chunk: int,
                     normalize: int = 1, eps: float = 1e-6, gamma: Optional[Sequence[float]] = None,
                     prf_w: Optional[torch.Tensor] = None, init_S: Optional[torch.Tensor] = None,
                     init_Z: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                     final_S: Optional[torch.Tensor] = None, final_Z: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None, events=None, layout: str = "bhtd",
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """o = chunkwise causal linear attention of q, k, v on the GPU (C ABI call).

    layout "bhtd": q, k, v, o are [B, H, T, d]; "bthd": [B, T, H, d]. o is allocated in
    out_dtype (float32, or bfloat16 = the fp32 result rounded to nearest even) unless given.
    events: optional sequence of 4 torch.cuda.Event (timing enabled) recorded at the phase
    boundaries through lin_attn_prefill_profiled."""
    if layout == "bhtd":
        B, H, T, d_k = q.shape
        lay = LA_LAYOUT_BHTD
    elif layout == "bthd":
        B, T, H, d_k = q.shape
        lay = LA_LAYOUT_BTHD
    else:
        raise ValueError(f"layout must be 'bhtd' or 'bthd', not {layout!r}")
    d_v = v.shape[-1]
    n_psi = prf_w.shape[1] if prf_w is not None else d_k
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError(f"q, k, v must be contiguous ({layout})")
    if o is None:
        shape = (B, H, T, d_v) if lay == LA_LAYOUT_BHTD else (B, T, H, d_v)
        o = torch.empty(shape, dtype=out_dtype, device=q.device)
    desc = prefill_desc(B, H, T, d_k, d_v, n_psi, chunk, psi, normalize, eps, _dtype_code(q), _dtype_code(o), lay)
    ws_bytes = workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    g = _gamma_array(gamma, H)
    args = [ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), g, _ptr(prf_w), _ptr(init_S), _ptr(init_Z), _ptr(o),
            _ptr(final_S), _ptr(final_Z), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)]
    if events is None:
        st = load().lin_attn_prefill(*args)
    else:
        ev = (ctypes.c_void_p * 4)(*[e.cuda_event if e is not None else None for e in events])
        st = load().lin_attn_prefill_profiled(*args, ev)
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill")
    return o


def lin_attn_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, psi: int, chunk: int,
                             normalize: int = 1, eps: float = 1e-6, gamma: Optional[Sequence[float]] = None,
                             prf_w: Optional[torch.Tensor] = None, init_S: Optional[torch.Tensor] = None,
                             init_Z: Optional[torch.Tensor] = None, o: Optional[torch.Tensor] = None,
                             final_S: Optional[torch.Tensor] = None, final_Z: Optional[torch.Tensor] = None,
                             stream=None, layout: str = "bhtd") -> torch.Tensor:
    """lin_attn_prefill through lin_attn_prefill_noalloc: no workspace; the library's per-device
    scratch holds the summary records. o must be given by callers that allocate nothing."""
    if layout == "bhtd":
        B, H, T, d_k = q.shape
        lay = LA_LAYOUT_BHTD
    elif layout == "bthd":
        B, T, H, d_k = q.shape
        lay = LA_LAYOUT_BTHD
    else:
        raise ValueError(f"layout must be 'bhtd' or 'bthd', not {layout!r}")
    d_v = v.shape[-1]
    n_psi = prf_w.shape[1] if prf_w is not None else d_k
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError(f"q, k, v must be contiguous ({layout})")
    if o is None:
        shape = (B, H, T, d_v) if lay == LA_LAYOUT_BHTD else (B, T, H, d_v)
        o = torch.empty(shape, dtype=torch.float32, device=q.device)
    desc = prefill_desc(B, H, T, d_k, d_v, n_psi, chunk, psi, normalize, eps, _dtype_code(q), _dtype_code(o), lay)
    st = load().lin_attn_prefill_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H),
                                         _ptr(prf_w), _ptr(init_S), _ptr(init_Z), _ptr(o), _ptr(final_S),
                                         _ptr(final_Z), _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_noalloc")
    return o


def lin_attn_prefill_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor,
                            max_seqlen: int, *, psi: int, chunk: int, normalize: int = 1, eps: float = 1e-6,
                            gamma: Optional[Sequence[float]] = None, prf_w: Optional[torch.Tensor] = None,
                            init_S: Optional[torch.Tensor] = None, init_Z: Optional[torch.Tensor] = None,
                            o: Optional[torch.Tensor] = None, final_S: Optional[torch.Tensor] = None,
                            final_Z: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                            stream=None, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Prefill of N packed sequences: q, k, v [total, H, d]; cu_seqlens int32 [N + 1] on the device
    (sequence b is tokens cu_seqlens[b] .. cu_seqlens[b+1] - 1); max_seqlen >= every length.
    States are per sequence: [N, H, n_psi, d_v] and [N, H, n_psi]."""
    total, H, d_k = q.shape
    d_v = v.shape[-1]
    N = cu_seqlens.numel() - 1
    n_psi = prf_w.shape[1] if prf_w is not None else d_k
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be an int32 tensor on the inputs' device")
    for t in (q, k, v, cu_seqlens):
        if not t.is_contiguous():
            raise ValueError("q, k, v [total, H, d] and cu_seqlens must be contiguous")
    if o is None:
        o = torch.empty((total, H, d_v), dtype=out_dtype, device=q.device)
    desc = prefill_desc(N, H, max_seqlen, d_k, d_v, n_psi, chunk, psi, normalize, eps, _dtype_code(q),
                        _dtype_code(o), LA_LAYOUT_BTHD)
    ws_bytes = varlen_workspace_size(desc, total)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    g = _gamma_array(gamma, H)
    st = load().lin_attn_prefill_varlen(ctypes.byref(desc), _ptr(cu_seqlens), total, _ptr(q), _ptr(k), _ptr(v), g,
                                        _ptr(prf_w), _ptr(init_S), _ptr(init_Z), _ptr(o), _ptr(final_S),
                                        _ptr(final_Z), _ptr(workspace),
                                        0 if workspace is None else workspace.numel() * workspace.element_size(),
                                        _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_varlen")
    return o


def backward_workspace_size(desc: PrefillDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load().lin_attn_prefill_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_backward_workspace_size")
    return int(n.value)


def lin_attn_prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, *, psi: int,
                              chunk: int, normalize: int = 1, eps: float = 1e-6,
                              gamma: Optional[Sequence[float]] = None, prf_w: Optional[torch.Tensor] = None,
                              init_S: Optional[torch.Tensor] = None,
                              init_Z: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                              dv: Optional[torch.Tensor] = None, dinit_S: Optional[torch.Tensor] = None,
                              dinit_Z: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                              stream=None, layout: str = "bhtd"):
    """(dq, dk, dv) of L = sum dout . o for lin_attn_prefill with the same arguments (C ABI call).

    dout is float32 or bfloat16, laid out like o. Gradients are float32 in the layouts of q, k,
    v; dinit_S / dinit_Z are written when given. prf_w: the random-feature bank (its n_psi sets
    the state width)."""
    if layout == "bhtd":
        B, H, T, d_k = q.shape
        lay = LA_LAYOUT_BHTD
    elif layout == "bthd":
        B, T, H, d_k = q.shape
        lay = LA_LAYOUT_BTHD
    else:
        raise ValueError(f"layout must be 'bhtd' or 'bthd', not {layout!r}")
    d_v = v.shape[-1]
    for t in (q, k, v, dout):
        if not t.is_contiguous():
            raise ValueError(f"q, k, v, dout must be contiguous ({layout})")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    n_psi = prf_w.shape[1] if prf_w is not None else d_k
    desc = prefill_desc(B, H, T, d_k, d_v, n_psi, chunk, psi, normalize, eps, _dtype_code(q), _dtype_code(dout), lay)
    ws_bytes = backward_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = load().lin_attn_prefill_backward(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), _ptr(prf_w), _ptr(init_S),
        _ptr(init_Z), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dinit_S), _ptr(dinit_Z), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_backward")
    return dq, dk, dv


def backward_varlen_workspace_size(desc: PrefillDesc, total_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    st = load().lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(desc), int(total_tokens),
                                                                ctypes.byref(n))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_backward_varlen_workspace_size")
    return int(n.value)


def lin_attn_prefill_backward_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                                     cu_seqlens: torch.Tensor, max_seqlen: int, *, psi: int, chunk: int,
                                     normalize: int = 1, eps: float = 1e-6, gamma: Optional[Sequence[float]] = None,
                                     init_S: Optional[torch.Tensor] = None, init_Z: Optional[torch.Tensor] = None,
                                     dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                                     dv: Optional[torch.Tensor] = None, dinit_S: Optional[torch.Tensor] = None,
                                     dinit_Z: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                                     stream=None):
    """(dq, dk, dv) of L = sum dout . o for lin_attn_prefill_varlen with the same arguments: q, k, v,
    dout [total, H, d]; cu_seqlens int32 [N + 1] on the device. Gradients are float32 [total, H, d];
    dinit_S [N, H, d_k, d_v] / dinit_Z [N, H, d_k] are written when given."""
    total, H, d_k = q.shape
    d_v = v.shape[-1]
    N = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be an int32 tensor on the inputs' device")
    for t in (q, k, v, dout, cu_seqlens):
        if not t.is_contiguous():
            raise ValueError("q, k, v, dout [total, H, d] and cu_seqlens must be contiguous")
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device) if dv is None else dv
    desc = prefill_desc(N, H, max_seqlen, d_k, d_v, d_k, chunk, psi, normalize, eps, _dtype_code(q),
                        _dtype_code(dout), LA_LAYOUT_BTHD)
    ws_bytes = backward_varlen_workspace_size(desc, total)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = load().lin_attn_prefill_backward_varlen(
        ctypes.byref(desc), _ptr(cu_seqlens), total, _ptr(q), _ptr(k), _ptr(v), _gamma_array(gamma, H), None,
        _ptr(init_S), _ptr(init_Z), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dinit_S), _ptr(dinit_Z),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_backward_varlen")
    return dq, dk, dv


def gated_workspace_size(desc: PrefillDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load().lin_attn_prefill_gated_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_gated_workspace_size")
    return int(n.value)


def lin_attn_prefill_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_gate: torch.Tensor, *,
                           psi: int, chunk: int = 32, normalize: int = 0, eps: float = 1e-6,
                           init_S: Optional[torch.Tensor] = None, init_Z: Optional[torch.Tensor] = None,
                           o: Optional[torch.Tensor] = None, final_S: Optional[torch.Tensor] = None,
                           final_Z: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None, layout: str = "bhtd", out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Gated prefill: q, k, v and the fp32 log forget gates (laid out like k) in layout "bhtd"
    [B, H, T, d] or "bthd" [B, T, H, d]."""
    if layout == "bhtd":
        B, H, T, d_k = q.shape
        lay = LA_LAYOUT_BHTD
    elif layout == "bthd":
        B, T, H, d_k = q.shape
        lay = LA_LAYOUT_BTHD
    else:
        raise ValueError(f"layout must be 'bhtd' or 'bthd', not {layout!r}")
    d_v = v.shape[-1]
    if log_gate.dtype != torch.float32 or log_gate.shape != k.shape:
        raise ValueError("log_gate must be fp32 and shaped like k")
    for t in (q, k, v, log_gate):
        if not t.is_contiguous():
            raise ValueError(f"q, k, v, log_gate must be contiguous ({layout})")
    if o is None:
        shape = (B, H, T, d_v) if lay == LA_LAYOUT_BHTD else (B, T, H, d_v)
        o = torch.empty(shape, dtype=out_dtype, device=q.device)
    desc = prefill_desc(B, H, T, d_k, d_v, d_k, chunk, psi, normalize, eps, _dtype_code(q), _dtype_code(o), lay)
    ws_bytes = gated_workspace_size(desc)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = load().lin_attn_prefill_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate), _ptr(init_S),
                                       _ptr(init_Z), _ptr(o), _ptr(final_S), _ptr(final_Z), _ptr(workspace),
                                       0 if workspace is None else workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_prefill_gated")
    return o


def lin_attn_decode_step_gated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_gate: torch.Tensor,
                               S: torch.Tensor, Z: Optional[torch.Tensor], *, psi: int, normalize: int = 1,
                               eps: float = 1e-6, prf_w: Optional[torch.Tensor] = None,
                               o: Optional[torch.Tensor] = None, stream=None,
                               out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """One gated decode step: q, k, v [N, H, d], log_gate fp32 [N, H, n_psi]; S, Z in place."""
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    n_psi = S.shape[-2]
    if o is None:
        o = torch.empty((N, H, d_v), dtype=out_dtype, device=q.device)
    desc = DecodeDesc(N, H, d_k, d_v, n_psi, psi, normalize, eps, _dtype_code(q), _dtype_code(o))
    st = load().lin_attn_decode_step_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_gate),
                                           _ptr(prf_w), _ptr(S), _ptr(Z), _ptr(o), _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_decode_step_gated")
    return o


def lin_attn_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, S: torch.Tensor,
                         Z: Optional[torch.Tensor], *, psi: int, normalize: int = 1, eps: float = 1e-6,
                         gamma: Optional[Sequence[float]] = None, prf_w: Optional[torch.Tensor] = None,
                         o: Optional[torch.Tensor] = None, stream=None,
                         out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """One decode step for q, k, v [N, H, d]; S [N, H, n_psi, d_v], Z [N, H, n_psi] updated in place.
    o is out_dtype (float32, or bfloat16 = the fp32 result rounded to nearest even) unless given."""
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    n_psi = S.shape[-2]
    if o is None:
        o = torch.empty((N, H, d_v), dtype=out_dtype, device=q.device)
    desc = DecodeDesc(N, H, d_k, d_v, n_psi, psi, normalize, eps, _dtype_code(q), _dtype_code(o))
    g = _gamma_array(gamma, H)
    st = load().lin_attn_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), g, _ptr(prf_w), _ptr(S),
                                     _ptr(Z), _ptr(o), _stream(stream))
    if st != LA_OK:
        raise LinAttnError(st, "lin_attn_decode_step")
    return o


def prefill_workload(w: "workloads.Workload", inputs: dict, **kw) -> torch.Tensor:
    """Run lin_attn_prefill on a named workload's inputs (see inputs.make_prefill_inputs)."""
    g = inputs.get("gamma")
    return lin_attn_prefill(inputs["q"], inputs["k"], inputs["v"], psi=w.psi, chunk=w.chunk,
                            normalize=w.normalize, eps=w.eps, gamma=None if g is None else list(g),
                            prf_w=inputs.get("prf_w"), **kw)
