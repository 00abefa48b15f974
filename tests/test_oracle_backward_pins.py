"""Pins of the backward oracle (oracle.prefill_backward) against what the mathematics fixes,
independently of the adjoint sweeps it implements. CPU only.

- Central differences of the (already pinned) forward oracle, entry by entry, Richardson-
  extrapolated: the gradient of L = sum_t dout_t . o_t with respect to every entry of q, k, v
  and of the initial state, for every feature map, with and without decay and normalisation.
- Automatic differentiation (torch, fp64) of the masked quadratic form, a second definition
  of the forward result ("Linear Attention and Retentive Networks", parallel representation
  (A) and the causal linear-attention sum).
- Exact dyadic inputs (identity features, small integers, gamma in {1, 1/2}, no denominator):
  every intermediate value is exact, so the adjoint sweeps and autograd must agree bitwise.
- Invariants: causality (a zero upstream gradient past t0 leaves every gradient past t0 zero,
  and the gradients before t0 equal those of the sequence cut at t0) and linearity in dout.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

PSI = {"identity": oracle.PSI_IDENTITY, "elu1": oracle.PSI_ELU1, "prf": oracle.PSI_PRF,
       "prf_qshift": oracle.PSI_PRF_QSHIFT}


def _grid(a: np.ndarray, bits: int = 20) -> np.ndarray:
    """Round to multiples of 2^-bits, so that x +- 2^-7 is exact in fp32."""
    return np.round(a * 2.0 ** bits) / 2.0 ** bits


def _problem(psi: str, T: int, d_k: int, d_v: int, n_psi: int, seed: int):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, d_k)) * 0.5
    k = rng.standard_normal((T, d_k)) * 0.5
    if psi == "elu1":  # keep away from the kink of elu's derivative at 0
        q = np.sign(q) * (np.abs(q) + 0.1)
        k = np.sign(k) * (np.abs(k) + 0.1)
    if psi == "identity":  # positive features: a denominator bounded away from 0
        q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
    v = rng.standard_normal((T, d_v))
    w = None
    if psi in ("prf", "prf_qshift"):
        while True:
            w = _grid(rng.standard_normal((n_psi, d_k)))
            lin = _grid(q) @ w.T
            top2 = np.sort(lin, axis=1)[:, -2:]
            if np.all(top2[:, 1] - top2[:, 0] > 0.05):  # a unique query argmax, far from a tie
                break
    S0 = rng.standard_normal((n_psi, d_v)) * 0.3
    Z0 = np.abs(rng.standard_normal(n_psi)) * 0.3 + 0.1
    dout = rng.standard_normal((T, d_v))
    f32 = lambda a: torch.from_numpy(_grid(a).astype(np.float32))
    return dict(q=f32(q), k=f32(k), v=f32(v), w=None if w is None else f32(w), S0=S0, Z0=Z0, dout=dout)


def _loss(pb, psi, gamma, normalize, eps, n_psi, q=None, k=None, v=None, S0=None, Z0=None):
    o = oracle.prefill(pb["q"] if q is None else q, pb["k"] if k is None else k, pb["v"] if v is None else v,
                       PSI[psi], n_psi=n_psi, prf_w=pb["w"], gamma=[gamma], normalize=normalize, eps=eps,
                       S0=pb["S0"] if S0 is None else S0, Z0=pb["Z0"] if Z0 is None else Z0, nthreads=1)
    return float(np.sum(o * pb["dout"]))


def _fd_grad(pb, name, psi, gamma, normalize, eps, n_psi):
    """Richardson-extrapolated central differences, (4 D(h/2) - D(h)) / 3, error O(h^4)."""
    x0 = pb[name]
    is_t = isinstance(x0, torch.Tensor)
    base = x0.double().numpy() if is_t else x0
    g = np.zeros(base.shape)
    h = 2.0 ** -7
    for idx in np.ndindex(base.shape):
        def L(delta):
            x = base.copy()
            x[idx] += delta
            arg = torch.from_numpy(x.astype(np.float32)) if is_t else x
            if is_t:
                assert float(arg[idx]) == x[idx]  # the perturbation is exact in fp32
            return _loss(pb, psi, gamma, normalize, eps, n_psi, **{name: arg})
        d1 = (L(h) - L(-h)) / (2 * h)
        d2 = (L(h / 2) - L(-h / 2)) / h
        g[idx] = (4 * d2 - d1) / 3
    return g


@pytest.mark.parametrize("psi", list(PSI))
@pytest.mark.parametrize("gamma", [1.0, 0.8])
@pytest.mark.parametrize("normalize", [0, 1])
def test_gradients_match_finite_differences(psi, gamma, normalize):
    T, d_k, d_v = 6, 4, 3
    n_psi = 6 if psi.startswith("prf") else d_k
    eps = 1e-3
    pb = _problem(psi, T, d_k, d_v, n_psi, seed=11 + 3 * normalize + (gamma < 1))
    dq, dk, dv, dS0, dZ0 = oracle.prefill_backward(
        pb["q"], pb["k"], pb["v"], pb["dout"], PSI[psi], n_psi=n_psi, prf_w=pb["w"], gamma=[gamma],
        normalize=normalize, eps=eps, S0=pb["S0"], Z0=pb["Z0"], nthreads=1)
    for name, got in (("q", dq), ("k", dk), ("v", dv), ("S0", dS0), ("Z0", dZ0)):
        fd = _fd_grad(pb, name, psi, gamma, normalize, eps, n_psi)
        scale = max(np.abs(fd).max(), 1e-3)
        err = np.abs(got - fd).max() / scale
        assert err < 1e-6, (name, err, got, fd)
    if not normalize:
        assert np.all(dZ0 == 0.0)


def _features_t(x, psi, w):
    if psi == "identity":
        return x
    if psi == "elu1":
        return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))
    lin = x @ w.T - 0.5 * (x * x).sum(-1, keepdim=True)
    if psi == "prf_qshift":
        lin = lin - lin.max(-1, keepdim=True).values
    return torch.exp(lin) / np.sqrt(w.shape[0])


def _quadratic_t(q, k, v, S0, Z0, psi, gamma, normalize, eps, w):
    """The masked quadratic form with an initial state, in torch fp64 (differentiable)."""
    T = q.shape[0]
    fq = _features_t(q, psi, w)
    fk = _features_t(k, "prf" if psi == "prf_qshift" else psi, w)
    lag = torch.arange(T)[:, None] - torch.arange(T)[None, :]
    D = torch.where(lag >= 0, torch.tensor(gamma, dtype=torch.float64) ** lag.clamp(min=0).double(),
                    torch.zeros((), dtype=torch.float64))
    A = (fq @ fk.T) * D
    dec0 = torch.tensor(gamma, dtype=torch.float64) ** torch.arange(1, T + 1, dtype=torch.float64)
    num = A @ v + dec0[:, None] * (fq @ S0)
    if not normalize:
        return num
    den = A.sum(1) + dec0 * (fq @ Z0) + eps
    return num / den[:, None]


@pytest.mark.parametrize("psi", list(PSI))
@pytest.mark.parametrize("gamma,normalize", [(1.0, 1), (0.9, 1), (0.95, 0)])
def test_gradients_match_autograd_of_quadratic_form(psi, gamma, normalize):
    T, d_k, d_v = 48, 8, 6
    n_psi = 12 if psi.startswith("prf") else d_k
    eps = 1e-4
    pb = _problem(psi, T, d_k, d_v, n_psi, seed=5)
    ts = {n: pb[n].double().clone().requires_grad_(True) for n in ("q", "k", "v")}
    S0 = torch.from_numpy(pb["S0"]).requires_grad_(True)
    Z0 = torch.from_numpy(pb["Z0"]).requires_grad_(True)
    w = None if pb["w"] is None else pb["w"].double()
    o = _quadratic_t(ts["q"], ts["k"], ts["v"], S0, Z0, psi, gamma, normalize, eps, w)
    # the differentiated function is the oracle's forward result
    o_orc = oracle.prefill(pb["q"], pb["k"], pb["v"], PSI[psi], n_psi=n_psi, prf_w=pb["w"], gamma=[gamma],
                           normalize=normalize, eps=eps, S0=pb["S0"], Z0=pb["Z0"])
    np.testing.assert_allclose(o.detach().numpy(), o_orc, rtol=1e-11, atol=1e-12)
    (o * torch.from_numpy(pb["dout"])).sum().backward()
    got = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], pb["dout"], PSI[psi], n_psi=n_psi, prf_w=pb["w"],
                                  gamma=[gamma], normalize=normalize, eps=eps, S0=pb["S0"], Z0=pb["Z0"])
    ref = (ts["q"].grad, ts["k"].grad, ts["v"].grad, S0.grad, Z0.grad)
    for name, g, r in zip(("dq", "dk", "dv", "dS0", "dZ0"), got, ref):
        r = np.zeros_like(g) if r is None else r.numpy()  # Z0 is unused without a denominator
        scale = max(np.abs(r).max(), 1e-12)
        assert np.abs(g - r).max() <= 1e-10 * scale, (name, np.abs(g - r).max(), scale)


@pytest.mark.parametrize("gamma,T", [(1.0, 40), (0.5, 24)])
def test_exact_dyadic_gradients_bitwise(gamma, T):
    rng = np.random.default_rng(3)
    d_k, d_v = 4, 3
    ints = lambda shape: rng.integers(-2, 3, size=shape).astype(np.float64)
    q, k, v, dout = ints((T, d_k)), ints((T, d_k)), ints((T, d_v)), ints((T, d_v))
    S0 = ints((d_k, d_v))
    f32 = lambda a: torch.from_numpy(a.astype(np.float32))
    got = oracle.prefill_backward(f32(q), f32(k), f32(v), dout, oracle.PSI_IDENTITY, gamma=[gamma], normalize=0,
                                  S0=S0, Z0=np.zeros(d_k))
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v, S0)]
    o = _quadratic_t(ts[0], ts[1], ts[2], ts[3], torch.zeros(d_k, dtype=torch.float64), "identity", gamma, 0, 0.0,
                     None)
    (o * torch.from_numpy(dout)).sum().backward()
    for g, t in zip(got[:4], ts):
        assert np.array_equal(g, t.grad.numpy())
    assert np.all(got[4] == 0.0)


@pytest.mark.parametrize("psi,normalize", [("elu1", 1), ("prf", 1), ("identity", 0)])
def test_causality_and_cut(psi, normalize):
    T, t0, d_k, d_v = 40, 23, 8, 5
    n_psi = 16 if psi == "prf" else d_k
    pb = _problem(psi, T, d_k, d_v, n_psi, seed=8)
    dout = pb["dout"].copy()
    dout[t0:] = 0.0
    kw = dict(n_psi=n_psi, prf_w=pb["w"], gamma=[0.93], normalize=normalize, eps=1e-3, S0=pb["S0"], Z0=pb["Z0"])
    dq, dk, dv, dS0, dZ0 = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], dout, PSI[psi], **kw)
    assert np.all(dq[t0:] == 0.0) and np.all(dk[t0:] == 0.0) and np.all(dv[t0:] == 0.0)
    cut = oracle.prefill_backward(pb["q"][:t0], pb["k"][:t0], pb["v"][:t0], dout[:t0], PSI[psi], **kw)
    for a, b in zip((dq[:t0], dk[:t0], dv[:t0], dS0, dZ0), cut):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_linear_in_upstream_gradient():
    T, d_k, d_v = 30, 8, 5
    pb = _problem("elu1", T, d_k, d_v, d_k, seed=9)
    rng = np.random.default_rng(10)
    d1, d2 = rng.standard_normal((T, d_v)), rng.standard_normal((T, d_v))
    kw = dict(gamma=[0.9], normalize=1, eps=1e-3, S0=pb["S0"], Z0=pb["Z0"])
    g1 = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], d1, oracle.PSI_ELU1, **kw)
    g2 = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], d2, oracle.PSI_ELU1, **kw)
    g3 = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], 2.0 * d1 - 0.5 * d2, oracle.PSI_ELU1, **kw)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, 2.0 * a - 0.5 * b, rtol=1e-10, atol=1e-12)


def test_blocks_are_independent():
    """Two (batch, head) blocks in one call: each block's gradients are those of its own call."""
    T, d_k, d_v = 20, 8, 4
    a, b = _problem("elu1", T, d_k, d_v, d_k, seed=12), _problem("elu1", T, d_k, d_v, d_k, seed=13)
    st = lambda n: torch.stack([a[n], b[n]])
    kw = dict(normalize=1, eps=1e-3)
    both = oracle.prefill_backward(st("q"), st("k"), st("v"), np.stack([a["dout"], b["dout"]]), oracle.PSI_ELU1,
                                   gamma=[0.9, 0.8], S0=np.stack([a["S0"], b["S0"]]),
                                   Z0=np.stack([a["Z0"], b["Z0"]]), **kw)
    for i, (pb, g) in enumerate(((a, 0.9), (b, 0.8))):
        one = oracle.prefill_backward(pb["q"], pb["k"], pb["v"], pb["dout"], oracle.PSI_ELU1, gamma=[g],
                                      S0=pb["S0"], Z0=pb["Z0"], **kw)
        for x, y in zip(both, one):
            np.testing.assert_array_equal(x[i], y)
