"""Host-side checks of liblinattn.so that need no GPU.

The library must load, export every function include/linattn.h declares, and
reject invalid arguments with the documented status codes before anything is
enqueued (so these calls never reach the device). The workspace planner is a pure
host function.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from chunked_causal_linear_k1_amd import binding
from chunked_causal_linear_k1_amd.binding import (LA_BF16, LA_ERR_ALIGN, LA_ERR_NULL, LA_ERR_SHAPE,
                                                  LA_ERR_UNSUPPORTED, LA_ERR_VALUE, LA_ERR_WORKSPACE, LA_F32, LA_OK,
                                                  DecodeDesc, PrefillDesc)

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "linattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH), reason="liblinattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lin_attn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = binding.load()
    names = _declared_functions()
    assert set(names) == set(binding.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def test_status_strings_and_version():
    for s in range(8):
        msg = binding.status_string(s)
        assert isinstance(msg, str) and msg
    assert binding.status_string(0) == "ok"
    assert binding.status_string(99) == "unknown status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", binding.version())


def _desc(**kw):
    base = dict(B=1, H=2, T=1000, d_k=128, d_v=128, n_psi=128, chunk=64, psi=1, normalize=1, eps=1e-6,
                in_dtype=LA_BF16, out_dtype=LA_F32)
    base.update(kw)
    return PrefillDesc(**base)


def _ws(desc):
    n = ctypes.c_size_t(0)
    st = binding.load().lin_attn_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), LA_ERR_SHAPE), (dict(B=0), LA_ERR_SHAPE), (dict(H=-1), LA_ERR_SHAPE),
    (dict(d_k=0), LA_ERR_SHAPE), (dict(chunk=0), LA_ERR_SHAPE),
    (dict(n_psi=64), LA_ERR_SHAPE),                       # n_psi != d_k without PRF
    (dict(psi=5), LA_ERR_VALUE), (dict(normalize=2), LA_ERR_VALUE), (dict(eps=-1.0), LA_ERR_VALUE),
    (dict(eps=float("nan")), LA_ERR_VALUE), (dict(in_dtype=5), LA_ERR_VALUE),
    (dict(chunk=48), LA_ERR_UNSUPPORTED), (dict(d_k=96, d_v=96, n_psi=96), LA_ERR_UNSUPPORTED),
    (dict(out_dtype=LA_BF16), LA_OK),                      # bf16 output = RNE of the fp32 result
    (dict(out_dtype=LA_BF16, in_dtype=LA_F32, d_k=64, d_v=64, n_psi=64), LA_ERR_UNSUPPORTED),
    (dict(out_dtype=7), LA_ERR_VALUE),
    # token layout: [B, H, T, d] or [B, T, H, d]
    (dict(layout=1), LA_OK), (dict(layout=1, in_dtype=LA_F32, d_k=64, d_v=64, n_psi=64), LA_OK),
    (dict(layout=2), LA_ERR_VALUE), (dict(layout=-1), LA_ERR_VALUE),
    # one interleaved chunk of one head must fit a 32-bit buffer range: C * H * d * 4 < 2^31
    (dict(layout=1, H=32768, chunk=128), LA_ERR_UNSUPPORTED), (dict(layout=1, H=512, chunk=128), LA_OK),
    (dict(in_dtype=LA_F32, chunk=128), LA_ERR_UNSUPPORTED),
    (dict(), LA_OK), (dict(chunk=128), LA_OK), (dict(d_k=64, d_v=64, n_psi=64), LA_OK),
    (dict(in_dtype=LA_F32, d_k=64, d_v=64, n_psi=64, chunk=64), LA_OK),
    # state rows must be whole 16-byte groups (the scan moves 4 floats per access)
    (dict(in_dtype=LA_F32, d_k=30, d_v=30, n_psi=30, chunk=32, psi=0), LA_ERR_UNSUPPORTED),
    (dict(in_dtype=LA_F32, d_k=32, d_v=32, n_psi=32, chunk=32, psi=0), LA_OK),
    # positive random features: bf16 needs d 128, n_psi 128 or 256; chunks 32, 64, 128 (all
    # walked in 64-token steps)
    (dict(psi=2, n_psi=256), LA_OK), (dict(psi=2, n_psi=128), LA_OK),
    (dict(psi=2, n_psi=64), LA_ERR_UNSUPPORTED), (dict(psi=2, n_psi=256, chunk=128), LA_OK),
    (dict(psi=2, n_psi=256, chunk=32), LA_OK), (dict(psi=2, n_psi=256, chunk=16), LA_ERR_UNSUPPORTED),
    # bf16 identity / elu+1: chunks 32, 64, 128
    (dict(chunk=32), LA_OK), (dict(chunk=32, d_k=64, d_v=64, n_psi=64, psi=0), LA_OK),
    (dict(chunk=16), LA_ERR_UNSUPPORTED), (dict(chunk=256), LA_ERR_UNSUPPORTED),
    # the same features with the query-row shift; anything past it is not a feature map
    (dict(psi=3, n_psi=256), LA_OK), (dict(psi=3, n_psi=128), LA_OK), (dict(psi=3, n_psi=64), LA_ERR_UNSUPPORTED),
    (dict(psi=3, in_dtype=LA_F32, d_k=64, d_v=64, n_psi=96, chunk=32), LA_OK), (dict(psi=4), LA_ERR_VALUE),
    # the shift cancels only against the denominator: without one it is refused
    (dict(psi=3, n_psi=256, normalize=0), LA_ERR_UNSUPPORTED),
    (dict(psi=3, in_dtype=LA_F32, d_k=64, d_v=64, n_psi=96, chunk=32, normalize=0), LA_ERR_UNSUPPORTED),
])
def test_prefill_validation(kw, status):
    st, _ = _ws(_desc(**kw))
    assert st == status, (kw, st, binding.status_string(st))


def test_workspace_size_planner():
    st, n1 = _ws(_desc(T=1000))
    assert st == LA_OK and n1 > 0
    # one summary (n_psi*d_v + n_psi fp32) per segment per sequence
    E = 128 * 128 + 128
    assert n1 % (4 * E) == 0
    st, n_big = _ws(_desc(T=131035, H=64, chunk=128, psi=0, normalize=0))
    assert st == LA_OK and n_big % (4 * E) == 0
    segs = n_big // (4 * E) // 64
    assert 1 <= segs <= 1024
    # 128k x 64 heads: 32 segments of 4096 tokens (sub-segments would pass 2048 workgroups)
    assert segs == 32
    # segments of at least 2048 tokens unless that leaves fewer than 256 workgroups:
    # the 8k x 64-sequence shape gets 4 segments of 2048 tokens (256 workgroups), whose
    # summaries are folded as two 1024-token records each (the workspace holds them all)
    st, n8 = _ws(_desc(B=4, H=16, T=8192))
    assert st == LA_OK and n8 == 4 * E * 64 * 4 * 2
    # the same with PRF features (n_psi 256) at 4k x 128 sequences: 2 segments, 2 records each
    Ep = 256 * 128 + 256
    st, n4 = _ws(_desc(B=8, H=16, T=4096, n_psi=256, psi=2))
    assert st == LA_OK and n4 == 4 * Ep * 128 * 2 * 2
    # fp32 inputs keep one record per segment
    Ef = 64 * 64 + 64
    st, n8f = _ws(_desc(B=4, H=16, T=8192, d_k=64, d_v=64, n_psi=64, in_dtype=binding.LA_F32))
    assert st == LA_OK and n8f == 4 * Ef * 64 * 4
    # a single short sequence still gets one segment per chunk up to 256 workgroups
    st, n1s = _ws(_desc(B=1, H=1, T=4096))
    assert st == LA_OK and n1s == 4 * E * 64
    # never more segments than chunks
    st, n_small = _ws(_desc(T=1, H=1))
    assert st == LA_OK and n_small == 4 * E
    # chunks of 32 tokens: segments hold an even number of chunks (whole 64-token steps); one
    # 100-token sequence gets 2 segments of 2 chunks, not 4 of 1
    st, n32 = _ws(_desc(B=1, H=1, T=100, chunk=32))
    assert st == LA_OK and n32 == 2 * 4 * E
    assert binding.load().lin_attn_prefill_workspace_size(None, None) == LA_ERR_NULL


def test_prefill_rejects_bad_pointers_before_launch():
    lib = binding.load()
    d = _desc()
    _, ws = _ws(d)
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    odd = ctypes.c_void_p((1 << 20) + 4)
    call = lambda q, k, v, o, w, wb, prf=None: lib.lin_attn_prefill(ctypes.byref(d), q, k, v, None, prf, None, None,
                                                                     o, None, None, w, wb, None)
    assert call(None, fake, fake, fake, fake, ws) == LA_ERR_NULL
    assert call(fake, fake, fake, None, fake, ws) == LA_ERR_NULL
    assert call(odd, fake, fake, fake, fake, ws) == LA_ERR_ALIGN
    assert call(fake, fake, fake, fake, None, ws) == LA_ERR_WORKSPACE
    assert call(fake, fake, fake, fake, fake, ws - 1) == LA_ERR_WORKSPACE
    # gamma outside (0, 1]
    bad_gamma = (ctypes.c_float * 2)(0.5, 1.5)
    assert lib.lin_attn_prefill(ctypes.byref(d), fake, fake, fake, bad_gamma, None, None, None, fake, None, None,
                                fake, ws, None) == LA_ERR_VALUE
    zero_gamma = (ctypes.c_float * 2)(0.0, 1.0)
    assert lib.lin_attn_prefill(ctypes.byref(d), fake, fake, fake, zero_gamma, None, None, None, fake, None, None,
                                fake, ws, None) == LA_ERR_VALUE
    # PRF needs its bank
    dp = _desc(psi=2, n_psi=256)
    st, wsp = _ws(dp)
    if st == LA_OK:
        assert lib.lin_attn_prefill(ctypes.byref(dp), fake, fake, fake, None, None, None, None, fake, None, None,
                                    fake, wsp, None) == LA_ERR_NULL


def test_varlen_rejects_bad_arguments_before_launch():
    lib = binding.load()
    d = _desc(B=3, T=700, layout=1)   # 3 packed sequences, longest 700 tokens
    ws = 1 << 30
    fake = ctypes.c_void_p(1 << 20)
    cu = ctypes.c_void_p(1 << 21)

    def call(desc=d, cu_=cu, total=1200, q=fake, o=fake, w=fake, wb=ws):
        return lib.lin_attn_prefill_varlen(ctypes.byref(desc), cu_, total, q, fake, fake, None, None, None, None, o,
                                           None, None, w, wb, None)
    assert call(cu_=None) == LA_ERR_NULL
    assert call(total=-1) == LA_ERR_SHAPE
    assert call(cu_=ctypes.c_void_p((1 << 21) + 2)) == LA_ERR_ALIGN   # int32 offsets: 4-byte aligned
    assert call(desc=_desc(B=3, T=700, layout=0)) == LA_ERR_VALUE    # packed tokens interleave the heads
    assert call(q=None) == LA_ERR_NULL
    assert call(w=None) == LA_ERR_WORKSPACE
    n = ctypes.c_size_t(0)
    assert lib.lin_attn_prefill_varlen_workspace_size(ctypes.byref(d), -1, ctypes.byref(n)) == LA_ERR_SHAPE
    assert lib.lin_attn_prefill_varlen_workspace_size(ctypes.byref(d), 1200, None) == LA_ERR_NULL


def test_varlen_planner():
    """Packed batches: segments of a fixed token count sized from the batch total (at least 2048
    tokens; about 2048 non-empty workgroups), one summary per (sequence, head, segment)."""
    lib = binding.load()
    E = 128 * 128 + 128

    def ws(total, **kw):
        n = ctypes.c_size_t(0)
        st = lib.lin_attn_prefill_varlen_workspace_size(ctypes.byref(_desc(layout=1, **kw)), total, ctypes.byref(n))
        assert st == LA_OK, binding.status_string(st)
        return n.value
    # 32 sequences x 32 heads, longest 16372, 259406 tokens: 8.3M token-heads / 2048 -> 4096-token segments
    assert ws(259406, B=32, H=32, T=16372, chunk=128, psi=0, normalize=0) == 32 * 32 * 4 * E * 4
    # small batches keep segments of 2048 tokens
    assert ws(3000, B=3, H=2, T=1000, chunk=64) == 3 * 2 * 1 * E * 4
    assert ws(30000, B=3, H=2, T=20000, chunk=64) == 3 * 2 * 10 * E * 4
    # an empty batch still plans one segment per sequence
    assert ws(0, B=3, H=2, T=1, chunk=64) == 3 * 2 * 1 * E * 4


def test_gated_validation_and_workspace():
    lib = binding.load()

    def ws(**kw):
        n = ctypes.c_size_t(0)
        st = lib.lin_attn_prefill_gated_workspace_size(ctypes.byref(_desc(**kw)), ctypes.byref(n))
        return st, n.value
    base = dict(chunk=32, psi=0, normalize=0)
    st, n = ws(**base)
    assert st == LA_OK
    # one record per segment: S, Z and the segment's per-row decay
    E = 128 * 128 + 2 * 128
    assert n % (4 * E) == 0
    for kw in (dict(chunk=64), dict(chunk=16), dict(psi=2, n_psi=256), dict(d_v=64), dict(d_k=96, d_v=96, n_psi=96)):
        assert ws(**{**base, **kw})[0] == LA_ERR_UNSUPPORTED, kw
    assert ws(**{**base, "psi": 1, "normalize": 1, "d_k": 64, "d_v": 64, "n_psi": 64})[0] == LA_OK
    assert ws(**{**base, "in_dtype": LA_F32, "layout": 1})[0] == LA_OK
    # the 4 x 16 x 8192 gated shape: 4 segments of 2048 tokens per sequence, summarised as two
    # 1024-token records each in bf16 (the workspace holds them all); fp32 inputs keep one
    st, n8 = ws(**{**base, "B": 4, "H": 16, "T": 8192})
    assert st == LA_OK and n8 == 4 * E * 64 * 4 * 2
    st, n8f = ws(**{**base, "B": 4, "H": 16, "T": 8192, "in_dtype": LA_F32})
    assert st == LA_OK and n8f == 4 * E * 64 * 4
    d = _desc(**base)
    fake, odd = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 4)
    call = lambda g, w=fake: lib.lin_attn_prefill_gated(ctypes.byref(d), fake, fake, fake, g, None, None, fake, None,
                                                        None, w, n, None)
    assert call(None) == LA_ERR_NULL
    assert call(odd) == LA_ERR_ALIGN
    assert call(fake, None) == LA_ERR_WORKSPACE
    dd = DecodeDesc(2, 2, 64, 64, 64, 1, 1, 1e-6, LA_BF16, LA_F32)
    assert lib.lin_attn_decode_step_gated(ctypes.byref(dd), fake, fake, fake, None, None, fake, fake, fake,
                                          None) == LA_ERR_NULL


def test_backward_validation_and_workspace():
    """Host-side checks of lin_attn_prefill_backward: supported shapes, workspace size, NULL and
    alignment errors and a gamma outside (0, 1] are all reported before anything is launched."""
    lib = binding.load()

    def ws(**kw):
        n = ctypes.c_size_t(0)
        st = lib.lin_attn_prefill_backward_workspace_size(ctypes.byref(_desc(**kw)), ctypes.byref(n))
        return st, n.value
    base = dict(B=2, H=4, T=1000, chunk=64, psi=1, normalize=1)
    st, n = ws(**base)
    assert st == LA_OK
    fwd = ctypes.c_size_t(0)
    assert lib.lin_attn_prefill_workspace_size(ctypes.byref(_desc(**base)), ctypes.byref(fwd)) == LA_OK
    # two segment-record regions plus 1/den and dden per token-head
    assert n == 2 * fwd.value + 2 * 4 * 1000 * 8
    st0, n0 = ws(**{**base, "normalize": 0})
    assert st0 == LA_OK and n0 == 2 * fwd.value
    assert ws(**{**base, "chunk": 128, "psi": 0})[0] == LA_OK
    assert ws(**{**base, "layout": 1})[0] == LA_OK
    assert ws(**{**base, "chunk": 32})[0] == LA_OK
    # fp32 inputs and bf16 at d = 64 take the vector-ALU sweeps: where the fp32 (or bf16) forward runs
    # and one step's tiles plus the state fit in LDS (random features up to n_psi = 128 at d = 128)
    for kw in (dict(d_k=64, d_v=64, n_psi=64), dict(d_k=64, d_v=64, n_psi=64, chunk=128),
               dict(in_dtype=LA_F32, chunk=32), dict(in_dtype=LA_F32, d_k=64, d_v=64, n_psi=64),
               dict(in_dtype=LA_F32, chunk=16, psi=0), dict(in_dtype=LA_F32, chunk=32, psi=2, n_psi=128),
               dict(in_dtype=LA_F32, chunk=32, psi=3, n_psi=128), dict(in_dtype=LA_F32, psi=2, n_psi=256, d_k=64,
                                                                     d_v=64, chunk=16)):
        st_, nb = ws(**{**base, **kw})
        assert st_ == LA_OK, kw
        f_ = ctypes.c_size_t(0)
        assert lib.lin_attn_prefill_workspace_size(ctypes.byref(_desc(**{**base, **kw})), ctypes.byref(f_)) == LA_OK
        tok = 2 * 4 * base["B"] * base["H"] * base["T"]
        if kw.get("in_dtype") == LA_F32:
            # two record regions of at least one record per sequence (the fp32 forward may plan its
            # own chunking for latency, so its workspace is not the backward's half)
            d_v, n_psi = kw.get("d_v", 128), kw.get("n_psi", 128)
            assert nb >= 2 * base["B"] * base["H"] * (n_psi * d_v + n_psi) * 4 + tok, kw
        else:
            assert nb == 2 * f_.value + tok, kw
    for kw in (dict(chunk=16), dict(in_dtype=LA_F32), dict(psi=2, n_psi=64), dict(psi=2, n_psi=256, chunk=16),
               dict(in_dtype=LA_F32, chunk=32, psi=2, n_psi=256), dict(in_dtype=LA_F32, chunk=128),
               dict(d_k=96, d_v=96, n_psi=96)):
        assert ws(**{**base, **kw})[0] == LA_ERR_UNSUPPORTED, kw
    # random features: one record per 64-token step (two regions), 1/den and dden per token-head,
    # and the bank transposed
    for npsi in (128, 256):
        for psi in (2, 3):
            st_, nb = ws(**{**base, "psi": psi, "n_psi": npsi})
            steps = -(-base["T"] // 64)
            recs = 2 * base["B"] * base["H"] * steps * (npsi * 128 + npsi) * 4
            tok = 2 * 4 * base["B"] * base["H"] * base["T"] if base.get("normalize", 1) else 0
            assert st_ == LA_OK and nb == recs + tok + base["H"] * npsi * 128 * 2, (psi, npsi, nb)
    assert ws(**{**base, "psi": 3, "n_psi": 256, "normalize": 0})[0] == LA_ERR_UNSUPPORTED
    d = _desc(**base)
    fake, odd = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 4)

    def call(q=fake, dout=fake, dq=fake, w=fake, gamma=None, size=n, desc=d, prf=None):
        return lib.lin_attn_prefill_backward(ctypes.byref(desc), q, fake, fake, gamma, prf, None, None, dout, dq, fake,
                                             fake, None, None, w, size, None)
    assert call(q=None) == LA_ERR_NULL
    assert call(dout=None) == LA_ERR_NULL
    assert call(dq=odd) == LA_ERR_ALIGN
    assert call(w=None) == LA_ERR_WORKSPACE
    assert call(size=n - 16) == LA_ERR_WORKSPACE
    assert call(gamma=(ctypes.c_float * 4)(1.0, 0.5, 0.0, 1.0)) == LA_ERR_VALUE
    dp = _desc(**{**base, "psi": 2, "n_psi": 256})
    _, nbp = ws(**{**base, "psi": 2, "n_psi": 256})
    assert call(desc=dp, size=nbp) == LA_ERR_NULL  # random features without the bank
    assert call(desc=dp, size=nbp, prf=odd) == LA_ERR_ALIGN


def test_backward_varlen_validation_and_workspace():
    """lin_attn_prefill_backward_varlen: workspace sized by the packed token count (the forward
    varlen plan twice plus 1/den and dden per token-head), and its argument errors before launch."""
    lib = binding.load()
    base = dict(B=5, H=4, T=3000, chunk=64, psi=1, normalize=1, layout=1)
    total = 4321
    n, fwd = ctypes.c_size_t(0), ctypes.c_size_t(0)
    d = _desc(**base)
    assert lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(d), total, ctypes.byref(n)) == LA_OK
    assert lib.lin_attn_prefill_varlen_workspace_size(ctypes.byref(d), total, ctypes.byref(fwd)) == LA_OK
    assert n.value == 2 * fwd.value + 2 * 4 * total * 4
    assert lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(d), -1, ctypes.byref(n)) == LA_ERR_SHAPE
    assert lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(d), total, None) == LA_ERR_NULL
    d32 = _desc(**{**base, "in_dtype": LA_F32})
    assert lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(d32), total,
                                                               ctypes.byref(n)) == LA_ERR_UNSUPPORTED
    lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(d), total, ctypes.byref(n))
    fake, odd = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 2)

    def call(desc=d, cu=fake, tot=total, q=fake, w=fake, size=n.value):
        return lib.lin_attn_prefill_backward_varlen(ctypes.byref(desc), cu, tot, q, fake, fake, None, None, None,
                                                    None, fake, fake, fake, fake, None, None, w, size, None)
    assert call(cu=None) == LA_ERR_NULL
    assert call(cu=odd) == LA_ERR_ALIGN
    assert call(tot=-1) == LA_ERR_SHAPE
    assert call(desc=_desc(**{**base, "layout": 0})) == LA_ERR_VALUE
    assert call(q=None) == LA_ERR_NULL
    assert call(size=n.value - 16) == LA_ERR_WORKSPACE
    dp = _desc(**{**base, "psi": 2, "n_psi": 256})  # random features: fixed-length batches only
    assert lib.lin_attn_prefill_backward_varlen_workspace_size(ctypes.byref(dp), total,
                                                               ctypes.byref(n)) == LA_ERR_UNSUPPORTED


def test_decode_validation():
    lib = binding.load()
    fake = ctypes.c_void_p(1 << 20)

    def call(desc, Z=fake, prf=None, S=fake):
        return lib.lin_attn_decode_step(ctypes.byref(desc), fake, fake, fake, None, prf, S, Z, fake, None)

    ok = dict(N=32, H=64, d_k=128, d_v=128, n_psi=128, psi=1, normalize=1, eps=1e-6, in_dtype=LA_BF16,
              out_dtype=LA_F32)
    assert call(DecodeDesc(**dict(ok, N=0))) == LA_ERR_SHAPE
    assert call(DecodeDesc(**dict(ok, psi=7))) == LA_ERR_VALUE
    assert call(DecodeDesc(**dict(ok, d_k=96, d_v=96, n_psi=96))) == LA_ERR_UNSUPPORTED
    assert call(DecodeDesc(**ok), Z=None) == LA_ERR_NULL
    assert call(DecodeDesc(**ok), S=None) == LA_ERR_NULL
    assert call(DecodeDesc(**dict(ok, psi=2, n_psi=256))) == LA_ERR_NULL  # PRF without bank
    assert call(DecodeDesc(**dict(ok, psi=3, n_psi=256, normalize=0)), prf=fake) == LA_ERR_UNSUPPORTED
    assert call(DecodeDesc(**ok), S=ctypes.c_void_p((1 << 20) + 8)) == LA_ERR_ALIGN
    assert lib.lin_attn_decode_step(None, fake, fake, fake, None, None, fake, fake, fake, None) == LA_ERR_NULL
    # bf16 output: with bf16 inputs only (as in prefill), an unknown dtype is a value error
    assert call(DecodeDesc(**dict(ok, out_dtype=LA_BF16, in_dtype=LA_F32))) == LA_ERR_UNSUPPORTED
    assert call(DecodeDesc(**dict(ok, out_dtype=7))) == LA_ERR_VALUE
    assert call(DecodeDesc(**dict(ok, out_dtype=LA_BF16)), S=ctypes.c_void_p((1 << 20) + 8)) == LA_ERR_ALIGN


def test_decay_head_limit():
    """Per-head decays travel by value in the launch arguments, at most LA_MAX_DECAY_HEADS = 256
    of them: 257 heads with gamma are rejected (prefill, backward, decode) before any launch. The
    accepted cases (256 heads with gamma, 257 without) are shown to pass the gamma check by the
    check that follows it, a workspace of zero bytes, so nothing is launched on these fake
    pointers."""
    lib = binding.load()
    fake = ctypes.c_void_p(1 << 20)
    g256 = (ctypes.c_float * 256)(*([0.99] * 256))
    g257 = (ctypes.c_float * 257)(*([0.99] * 257))
    for H, g, want in ((256, g256, LA_ERR_WORKSPACE), (257, g257, LA_ERR_UNSUPPORTED), (257, None, LA_ERR_WORKSPACE)):
        d = _desc(B=1, H=H, T=100, chunk=64, psi=0, normalize=0)
        got = lib.lin_attn_prefill(ctypes.byref(d), fake, fake, fake, g, None, None, None, fake, None, None, fake, 0,
                                   None)
        assert got == want, ("prefill", H, got)
        gotb = lib.lin_attn_prefill_backward(ctypes.byref(d), fake, fake, fake, g, None, None, None, fake, fake, fake,
                                             fake, None, None, fake, 0, None)
        assert gotb == want, ("backward", H, gotb)
    dd = DecodeDesc(N=1, H=257, d_k=128, d_v=128, n_psi=128, psi=0, normalize=0, eps=1e-6, in_dtype=LA_BF16,
                    out_dtype=LA_F32)
    assert lib.lin_attn_decode_step(ctypes.byref(dd), fake, fake, fake, g257, None, fake, None, fake,
                                    None) == LA_ERR_UNSUPPORTED


def test_sequence_count_beyond_grid_y_extent():
    """B x H is not capped at 65535: sequences go on the grid's x extent (2^31 - 1)."""
    lib = binding.load()
    for B, H in ((70000, 1), (4096, 64)):
        d = _desc(B=B, H=H, T=100, chunk=64, psi=0, normalize=0)
        nbytes = ctypes.c_size_t(0)
        assert lib.lin_attn_prefill_workspace_size(ctypes.byref(d), ctypes.byref(nbytes)) == 0, (B, H)
        assert nbytes.value > 0


def test_scan_depth_validation():
    """lin_attn_scan_depth checks its arguments before any launch."""
    lib = binding.load()
    fake = ctypes.c_void_p(1 << 20)
    assert lib.lin_attn_scan_depth(8, None, fake, None) == LA_ERR_NULL
    assert lib.lin_attn_scan_depth(8, fake, None, None) == LA_ERR_NULL
    assert lib.lin_attn_scan_depth(0, fake, fake, None) == LA_ERR_SHAPE
    assert lib.lin_attn_scan_depth(65536, fake, fake, None) == LA_ERR_SHAPE
    assert lib.lin_attn_scan_depth(8, ctypes.c_void_p((1 << 20) + 8), fake, None) == LA_ERR_ALIGN
