"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle (oracle/linattn_oracle.c through oracle/__init__.py)
against something other than itself:
  * hand-worked examples (tests/golden/handworked.txt),
  * the masked quadratic ("parallel") form on tiny inputs (oracle/brute.py),
  * exact dyadic arithmetic, where recurrence, quadratic form and the chunked
    method under three scan orders must agree bit for bit,
  * closed forms (constant values, zero inputs, PRF expectation),
  * invariants (causality, ragged prefixes, state hand-off, decode = prefill).
None of these tests needs a GPU.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked.txt")


# ----------------------------------------------------------------------------- helpers
def _parse_golden(path=GOLDEN):
    cases, cur = {}, None
    for raw in open(path):
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = cases.setdefault(rest.strip(), {})
            continue
        if "|" in rest or len(rest.split()) > 1:
            rows = [[float(x) for x in r.split()] for r in rest.split("|")]
            cur[key] = np.array(rows, dtype=np.float64)
        else:
            tok = rest.strip()
            try:
                cur[key] = float(tok)
            except ValueError:
                cur[key] = tok
    return cases


def _f32(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.float32)


PSI = {"identity": oracle.PSI_IDENTITY, "elu1": oracle.PSI_ELU1, "prf": oracle.PSI_PRF,
       "prf_qshift": oracle.PSI_PRF_QSHIFT}


# ----------------------------------------------------------------------------- golden
def test_golden_retention_identity():
    c = _parse_golden()["retention_identity"]
    q, k, v = (_f32(c[n])[None] for n in ("q", "k", "v"))
    o, S, Z = oracle.prefill(q, k, v, oracle.PSI_IDENTITY, gamma=[c["gamma"]], normalize=0,
                             want_state=True)
    np.testing.assert_array_equal(o[0], c["o_plain"])
    np.testing.assert_array_equal(S[0], c["S_final"])
    np.testing.assert_array_equal(Z[0], c["Z_final"][0])
    on = oracle.prefill(q, k, v, oracle.PSI_IDENTITY, gamma=[c["gamma"]], normalize=1, eps=0.0)
    np.testing.assert_allclose(on[0], c["o_normalized_eps0"], rtol=1e-15, atol=0)


def test_golden_elu1_scalar():
    c = _parse_golden()["elu1_scalar"]
    q, k, v = (_f32(c[n])[None] for n in ("q", "k", "v"))
    o = oracle.prefill(q, k, v, oracle.PSI_ELU1, normalize=1, eps=0.0)
    np.testing.assert_allclose(o[0], c["o_normalized_eps0"], rtol=1e-15, atol=0)


def test_golden_prf_vector():
    c = _parse_golden()["prf_vector"]
    w = c["w"]  # [m, d_k]
    phi = oracle.feature(np.array([c["x"]]), oracle.PSI_PRF, n_psi=w.shape[0], w=w)
    np.testing.assert_allclose(phi, c["phi"][0], rtol=1e-15)


# ----------------------------------------------------------------------------- feature maps
def test_elu1_values():
    x = np.array([0.0, 1.0, 2.5, -math.log(2.0), -1e-300, 3e-8])
    got = oracle.feature(x, oracle.PSI_ELU1)
    # elu(x)+1 = x+1 for x > 0, e^x for x <= 0; e^(-ln 2) = 1/2
    np.testing.assert_allclose(got, [1.0, 2.0, 3.5, 0.5, 1.0, 1.0 + 3e-8], rtol=1e-15)


def test_identity_feature():
    x = np.array([-3.0, 0.0, 7.25])
    np.testing.assert_array_equal(oracle.feature(x, oracle.PSI_IDENTITY), x)


def test_prf_zero_input_and_zero_bank():
    rng = np.random.default_rng(5)
    m, d = 16, 8
    w = rng.standard_normal((m, d))
    # psi(0) = exp(0 - 0)/sqrt(m) in every coordinate
    np.testing.assert_allclose(oracle.feature(np.zeros(d), oracle.PSI_PRF, m, w), np.full(m, m ** -0.5),
                               rtol=1e-15)
    # with an all-zero bank, psi(x) = exp(-|x|^2/2)/sqrt(m)
    x = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.feature(x, oracle.PSI_PRF, m, np.zeros((m, d))),
                               np.full(m, math.exp(-0.5 * float(x @ x)) / math.sqrt(m)), rtol=1e-14)


def test_prf_expectation_is_softmax_kernel():
    """E_W[psi(x).psi(y)] = exp(x.y) for Gaussian rows ("Linearized 2-Simplicial
    Attention", section 3.2, proved with the Gaussian moment-generating function).
    Monte-Carlo over m = 2^16 rows, checked within 6 standard errors."""
    rng = np.random.default_rng(11)
    d, m = 4, 1 << 16
    x = rng.standard_normal(d) * 0.4
    y = rng.standard_normal(d) * 0.4
    w = rng.standard_normal((m, d))
    fx = oracle.feature(x, oracle.PSI_PRF, m, w)
    fy = oracle.feature(y, oracle.PSI_PRF, m, w)
    per_row = fx * fy * m  # each row's unbiased estimate of exp(x.y)
    est = per_row.mean()
    se = per_row.std(ddof=1) / math.sqrt(m)
    assert abs(est - math.exp(float(x @ y))) < 6 * se, (est, math.exp(float(x @ y)), se)
    # the 1/sqrt(m) scale: dot product of features is the mean, not the sum
    assert abs(float(fx @ fy) - est) < 1e-12 * abs(est)


def test_qshift_largest_query_feature_is_one_over_sqrt_m():
    """The log-space shift of "Linearized 2-Simplicial Attention" (appendix B.2) subtracts the
    query row's largest log-feature, so that feature becomes exp(0) / sqrt(m) and every other
    is smaller; the ratios between features are those of the unshifted map."""
    rng = np.random.default_rng(3)
    m, d = 64, 8
    w = rng.standard_normal((m, d))
    for scale in (0.3, 3.0, 30.0):  # at 30 the unshifted features underflow or overflow in fp64
        x = rng.standard_normal(d) * scale
        f = oracle.feature(x, oracle.PSI_PRF_QSHIFT, m, w)
        assert np.all(np.isfinite(f)) and np.all(f > 0)
        assert abs(f.max() * math.sqrt(m) - 1.0) < 1e-15
        if scale < 10:
            g = oracle.feature(x, oracle.PSI_PRF, m, w)
            np.testing.assert_allclose(f / f.max(), g / g.max(), rtol=1e-12)


@pytest.mark.parametrize("gamma", [1.0, 0.9])
def test_qshift_cancels_without_eps(gamma):
    """The shift depends on the query row only and multiplies numerator and denominator alike:
    with eps = 0 the output equals that of the unshifted features."""
    T, d_k, d_v, m = 40, 8, 6, 24
    q, k = _rand((2, T, d_k), 5, 0.8), _rand((2, T, d_k), 6, 0.8)
    v = _rand((2, T, d_v), 7)
    w = _rand((1, m, d_k), 8)
    a = oracle.prefill(q, k, v, oracle.PSI_PRF_QSHIFT, n_psi=m, prf_w=w, gamma=[gamma, gamma], normalize=1, eps=0.0)
    b = oracle.prefill(q, k, v, oracle.PSI_PRF, n_psi=m, prf_w=w, gamma=[gamma, gamma], normalize=1, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)
    # the states are those of the keys, which take no shift
    _, Sa, Za = oracle.prefill(None, k, v, oracle.PSI_PRF_QSHIFT, n_psi=m, prf_w=w, want_state=True)
    _, Sb, Zb = oracle.prefill(None, k, v, oracle.PSI_PRF, n_psi=m, prf_w=w, want_state=True)
    assert np.array_equal(Sa, Sb) and np.array_equal(Za, Zb)


# ----------------------------------------------------------------------------- brute force
CASES = [
    # psi, gamma, normalize, T, d_k, d_v, n_psi, scale
    ("identity", 1.0, 0, 37, 8, 8, 8, 0.5),
    ("identity", 0.9, 0, 64, 8, 6, 8, 0.5),
    ("identity", 0.5, 1, 29, 4, 4, 4, 1.0),
    ("elu1", 1.0, 1, 64, 8, 8, 8, 1.0),
    ("elu1", 0.93, 1, 50, 6, 5, 6, 1.0),
    ("elu1", 1.0, 0, 17, 8, 8, 8, 1.0),
    ("prf", 1.0, 1, 40, 8, 8, 16, 0.6),
    ("prf", 0.95, 1, 33, 6, 4, 12, 0.6),
    ("prf_qshift", 1.0, 1, 40, 8, 8, 16, 0.6),
    ("prf_qshift", 0.95, 1, 33, 6, 4, 12, 1.5),
    ("prf_qshift", 0.9, 0, 21, 6, 4, 12, 1.0),
]


@pytest.mark.parametrize("psi,gamma,normalize,T,d_k,d_v,n_psi,scale", CASES)
def test_recurrence_matches_quadratic_form(psi, gamma, normalize, T, d_k, d_v, n_psi, scale):
    seed = hash((psi, gamma, T)) & 0xFFFF
    q = _rand((1, T, d_k), seed, scale)
    k = _rand((1, T, d_k), seed + 1, scale)
    v = _rand((1, T, d_v), seed + 2)
    w = _rand((n_psi, d_k), seed + 3) if psi.startswith("prf") else None
    eps = 1e-3
    o = oracle.prefill(q, k, v, PSI[psi], n_psi=n_psi, prf_w=None if w is None else w[None],
                       gamma=[gamma], normalize=normalize, eps=eps)[0]
    ref = brute.quadratic(oracle.as_f64(q[0]), oracle.as_f64(k[0]), oracle.as_f64(v[0]), PSI[psi],
                          gamma, normalize, eps, None if w is None else oracle.as_f64(w))
    np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


@pytest.mark.parametrize("psi", ["identity", "elu1", "prf", "prf_qshift"])
def test_initial_state_matches_quadratic_form(psi):
    T, d_k, d_v = 23, 6, 5
    n_psi = 10 if psi.startswith("prf") else d_k
    q, k = _rand((1, T, d_k), 1, 0.5), _rand((1, T, d_k), 2, 0.5)
    v = _rand((1, T, d_v), 3)
    w = _rand((n_psi, d_k), 4) if psi.startswith("prf") else None
    rng = np.random.default_rng(0)
    S0 = rng.standard_normal((n_psi, d_v))
    Z0 = np.abs(rng.standard_normal(n_psi)) + 1.0
    for normalize in (0, 1):
        o = oracle.prefill(q, k, v, PSI[psi], n_psi=n_psi, prf_w=None if w is None else w[None],
                           gamma=[0.8], normalize=normalize, eps=1e-3, S0=S0[None], Z0=Z0[None])[0]
        ref = brute.quadratic(oracle.as_f64(q[0]), oracle.as_f64(k[0]), oracle.as_f64(v[0]), PSI[psi], 0.8,
                              normalize, 1e-3, None if w is None else oracle.as_f64(w), S0=S0, Z0=Z0)
        np.testing.assert_allclose(o, ref, rtol=1e-11, atol=1e-11 * np.abs(ref).max())


# ----------------------------------------------------------------------------- exact dyadic arithmetic
def _int_inputs(T, d_k, d_v, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda d: torch.randint(lo, hi + 1, (1, T, d), generator=g).to(torch.float32)
    return mk(d_k), mk(d_k), mk(d_v)


@pytest.mark.parametrize("gamma,T", [(1.0, 200), (0.5, 31)])
@pytest.mark.parametrize("C", [4, 8, 16, 32])
def test_exact_dyadic_recurrence_equals_chunked_scans(gamma, T, C):
    """Every value is an exact dyadic rational, so the recurrence, the quadratic form
    and the chunked method under sequential, Hillis-Steele and Blelloch scan orders
    must agree bit for bit (the scan "is mathematically identical to sequential
    accumulation": "Log-Depth Chunked Linear-Attention Scan", Implementation notes),
    with the non-commutative decayed monoid when gamma = 1/2 and a ragged tail."""
    q, k, v = _int_inputs(T, 4, 3, -2, 2, seed=T * 100 + C)
    o, S, Z = oracle.prefill(q, k, v, oracle.PSI_IDENTITY, gamma=[gamma], normalize=0, want_state=True)
    qa, ka, va = (oracle.as_f64(x[0]) for x in (q, k, v))
    np.testing.assert_array_equal(o[0], brute.quadratic(qa, ka, va, 0, gamma, 0))
    for scan in ("sequential", "hillis_steele", "blelloch"):
        oc, info = chunked.chunked(qa, ka, va, 0, C, gamma, 0, scan=scan, return_info=True)
        np.testing.assert_array_equal(o[0], oc, err_msg=scan)
        np.testing.assert_array_equal(S[0], info["S"], err_msg=scan)
        np.testing.assert_array_equal(Z[0], info["Z"], err_msg=scan)
    # normalised with a dyadic eps: numerators and denominators are exact, so the quotients agree too
    on = oracle.prefill(q, k, v, oracle.PSI_IDENTITY, gamma=[gamma], normalize=1, eps=0.5)
    for scan in ("sequential", "hillis_steele", "blelloch"):
        np.testing.assert_array_equal(on[0], chunked.chunked(qa, ka, va, 0, C, gamma, 1, eps=0.5, scan=scan))


def test_exact_elu1_integer_features():
    # psi(x) = x + 1 for x in {1, 2} and psi(0) = e^0 = 1: all exact
    q, k, v = _int_inputs(77, 4, 4, 0, 2, seed=3)
    o = oracle.prefill(q, k, v, oracle.PSI_ELU1, normalize=1, eps=0.5)
    qa, ka, va = (oracle.as_f64(x[0]) for x in (q, k, v))
    np.testing.assert_array_equal(o[0], brute.quadratic(qa, ka, va, 1, 1.0, 1, 0.5))
    np.testing.assert_array_equal(o[0], chunked.chunked(qa, ka, va, 1, 16, 1.0, 1, eps=0.5))


@pytest.mark.parametrize("psi", ["prf", "prf_qshift"])
def test_chunked_prf_matches_recurrence(psi):
    """The chunked statement with random features, including the query-row shift (keys take
    no shift: only the query row's largest log-feature is subtracted), against the recurrence,
    with decay, a denominator and a ragged last chunk."""
    T, d_k, d_v, m, C = 45, 6, 5, 12, 8
    q, k = _rand((1, T, d_k), 31, 1.2), _rand((1, T, d_k), 32, 1.2)
    v = _rand((1, T, d_v), 33)
    w = _rand((m, d_k), 34)
    o = oracle.prefill(q, k, v, PSI[psi], n_psi=m, prf_w=w[None], gamma=[0.9], normalize=1, eps=1e-3)[0]
    oc = chunked.chunked(oracle.as_f64(q[0]), oracle.as_f64(k[0]), oracle.as_f64(v[0]), PSI[psi], C, 0.9, 1,
                         eps=1e-3, w=oracle.as_f64(w))
    np.testing.assert_allclose(oc, o, rtol=1e-11, atol=1e-11 * np.abs(o).max())


@pytest.mark.parametrize("n_chunks", [1, 2, 3, 5, 8, 16, 33, 128, 1024])
def test_scan_round_counts(n_chunks):
    """Hillis-Steele takes ceil(log2 N_C) rounds ("Log-Depth Chunked Linear-Attention
    Scan", Stage 1: observed rounds matched ceil(log2(number of chunks))); Blelloch takes
    an up-sweep and a down-sweep of that depth."""
    xs = [chunked.Summary(1.0, np.full((1, 1), float(i)), np.zeros(1)) for i in range(n_chunks)]
    _, r_hs = chunked.scan_hillis_steele(xs)
    _, r_bl = chunked.scan_blelloch(xs)
    depth = math.ceil(math.log2(n_chunks)) if n_chunks > 1 else 0
    assert r_hs == depth
    assert r_bl == 2 * depth


def test_blelloch_is_order_sensitive():
    """With gamma < 1 the monoid does not commute; combining in the wrong order must
    change the result (so the exactness test above really tests order)."""
    a = chunked.Summary(0.5, np.ones((1, 1)), np.zeros(1))
    b = chunked.Summary(0.5, 2 * np.ones((1, 1)), np.zeros(1))
    assert chunked.combine(a, b).S[0, 0] != chunked.combine(b, a).S[0, 0]


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("psi,gamma", [("elu1", 1.0), ("elu1", 0.9), ("prf", 0.97)])
def test_constant_values_give_constant_output(psi, gamma):
    """v_i = c for all i and eps = 0: o_t = c exactly (num = c * den), whatever the
    positive features and decay, provided Z decays like S."""
    T, d_k, d_v = 45, 6, 3
    n_psi = 9 if psi == "prf" else d_k
    q, k = _rand((1, T, d_k), 7, 0.7), _rand((1, T, d_k), 8, 0.7)
    c = np.array([1.5, -0.25, 3.0], dtype=np.float32)
    v = torch.tensor(np.tile(c, (1, T, 1)))
    w = _rand((1, n_psi, d_k), 9) if psi == "prf" else None
    o = oracle.prefill(q, k, v, PSI[psi], n_psi=n_psi, prf_w=w, gamma=[gamma], normalize=1, eps=0.0)
    np.testing.assert_allclose(o[0], np.tile(c.astype(np.float64), (T, 1)), rtol=1e-13)


def test_single_token():
    """T = 1: o_1 = v_1 w / (w + eps) with w = psi(q_1).psi(k_1) (elu+1 of 1 and 0.5 are 2 and 1.5)."""
    q = _f32([[[1.0, 0.5]]])
    k = _f32([[[0.5, 1.0]]])
    v = _f32([[[4.0, -2.0]]])
    w_ = 2.0 * 1.5 + 1.5 * 2.0
    o = oracle.prefill(q, k, v, oracle.PSI_ELU1, normalize=1, eps=0.25)
    np.testing.assert_allclose(o[0, 0], np.array([4.0, -2.0]) * w_ / (w_ + 0.25), rtol=1e-15)


def test_decay_of_old_tokens():
    """With identity features, gamma = 1/2, one key at t = 1 and zero keys after it,
    o_t = gamma^(t-1) (q_t.k_1) v_1."""
    T = 10
    q = torch.ones((1, T, 2))
    k = torch.zeros((1, T, 2)); k[0, 0] = torch.tensor([1.0, 2.0])
    v = torch.zeros((1, T, 1)); v[0, 0, 0] = 3.0
    o = oracle.prefill(q, k, v, oracle.PSI_IDENTITY, gamma=[0.5], normalize=0)
    np.testing.assert_array_equal(o[0, :, 0], [3.0 * 3.0 * 0.5 ** t for t in range(T)])


# ----------------------------------------------------------------------------- invariants
def test_causality_and_ragged_prefix():
    T, d = 60, 8
    q, k, v = _rand((2, T, d), 1), _rand((2, T, d), 2), _rand((2, T, d), 3)
    o = oracle.prefill(q, k, v, oracle.PSI_ELU1, gamma=[0.95, 0.9], normalize=1)
    # perturb the tail after t0: the head up to t0 is unchanged
    t0 = 37
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, t0:] += 1.0; k2[:, t0:] -= 0.5; v2[:, t0:] *= 3.0
    o2 = oracle.prefill(q2, k2, v2, oracle.PSI_ELU1, gamma=[0.95, 0.9], normalize=1)
    np.testing.assert_array_equal(o[:, :t0], o2[:, :t0])
    assert not np.allclose(o[:, t0:], o2[:, t0:])
    # a shorter sequence gives exactly the prefix of the longer one
    o3 = oracle.prefill(q[:, :t0].contiguous(), k[:, :t0].contiguous(), v[:, :t0].contiguous(),
                        oracle.PSI_ELU1, gamma=[0.95, 0.9], normalize=1)
    np.testing.assert_array_equal(o[:, :t0], o3)


def test_state_handoff_split_anywhere():
    T, d = 50, 6
    q, k, v = _rand((1, T, d), 4), _rand((1, T, d), 5), _rand((1, T, d), 6)
    o, S, Z = oracle.prefill(q, k, v, oracle.PSI_ELU1, gamma=[0.9], normalize=1, want_state=True)
    for t1 in (1, 17, 49):
        a = slice(0, t1); b = slice(t1, T)
        _, S1, Z1 = oracle.prefill(q[:, a].contiguous(), k[:, a].contiguous(), v[:, a].contiguous(),
                                   oracle.PSI_ELU1, gamma=[0.9], normalize=1, want_state=True)
        ob, S2, Z2 = oracle.prefill(q[:, b].contiguous(), k[:, b].contiguous(), v[:, b].contiguous(),
                                    oracle.PSI_ELU1, gamma=[0.9], normalize=1, S0=S1, Z0=Z1, want_state=True)
        np.testing.assert_allclose(ob, o[:, b], rtol=1e-13)
        np.testing.assert_allclose(S2, S, rtol=1e-13)
        np.testing.assert_allclose(Z2, Z, rtol=1e-13)


def test_decode_steps_equal_prefill():
    """Prefill of P tokens followed by n decode steps equals prefill of P + n tokens."""
    P, n, d = 30, 5, 8
    blocks = 3
    q, k, v = _rand((blocks, P + n, d), 10), _rand((blocks, P + n, d), 11), _rand((blocks, P + n, d), 12)
    gam = [0.99, 0.9, 1.0]
    o_full = oracle.prefill(q, k, v, oracle.PSI_ELU1, gamma=gam, normalize=1)
    _, S, Z = oracle.prefill(None, k[:, :P].contiguous(), v[:, :P].contiguous(), oracle.PSI_ELU1, gamma=gam,
                             normalize=1, want_state=True)
    S, Z = np.ascontiguousarray(S), np.ascontiguousarray(Z)
    for t in range(P, P + n):
        ot = oracle.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), S, Z,
                                oracle.PSI_ELU1, gamma=gam, normalize=1)
        np.testing.assert_allclose(ot, o_full[:, t], rtol=1e-13)


def test_per_block_gamma_and_bank():
    """Blocks are independent: a batched call equals per-block calls with that block's gamma and bank."""
    T, d, m = 20, 4, 6
    q, k, v = _rand((3, T, d), 20, 0.5), _rand((3, T, d), 21, 0.5), _rand((3, T, d), 22)
    w = _rand((2, m, d), 23)
    gam, heads = [0.9, 0.8, 1.0], [1, 0, 1]
    o = oracle.prefill(q, k, v, oracle.PSI_PRF, n_psi=m, prf_w=w, w_head=heads, gamma=gam)
    for b in range(3):
        ob = oracle.prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], oracle.PSI_PRF, n_psi=m,
                            prf_w=w[heads[b]:heads[b] + 1], gamma=[gam[b]])
        np.testing.assert_array_equal(o[b], ob[0])


def test_bf16_inputs_upcast_exactly():
    x = torch.tensor([[[1.0 + 2 ** -7, -3.0, 0.15625]]], dtype=torch.bfloat16)
    o = oracle.prefill(x, x, x, oracle.PSI_IDENTITY, normalize=0)
    xd = x.to(torch.float64).numpy()[0, 0]
    np.testing.assert_array_equal(o[0, 0], (xd @ xd) * xd)


# ----------------------------------------------------------------------------- gated recurrence
def _gates(shape, seed, lo=-3.0):
    """log forget gates in [lo, 0): log-sigmoid of a scaled Gaussian, fp32 (the values both
    sides receive)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * 2.0 + 1.0
    return torch.clamp(torch.nn.functional.logsigmoid(x), min=lo).to(torch.float32)


@pytest.mark.parametrize("psi,normalize,with_state", [("identity", 0, False), ("identity", 0, True),
                                                       ("elu1", 1, False), ("elu1", 1, True),
                                                       ("prf", 1, True)])
def test_gated_recurrence_matches_quadratic_form(psi, normalize, with_state):
    """S_t = diag(alpha_t) S_{t-1} + psi(k_t) v_t^T against the parallel form with the
    products of the gates between writer and reader ("Linear Attention and Retentive
    Networks", Data-Dependent Gating Mechanism)."""
    T, d_k, d_v = 45, 6, 5
    n_psi = 9 if psi == "prf" else d_k
    q, k = _rand((1, T, d_k), 21, 0.7), _rand((1, T, d_k), 22, 0.7)
    v = _rand((1, T, d_v), 23)
    w = _rand((n_psi, d_k), 24) if psi == "prf" else None
    lg = _gates((1, T, n_psi), 25)
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((n_psi, d_v)) if with_state else None
    Z0 = np.abs(rng.standard_normal(n_psi)) + 1.0 if with_state else None
    o = oracle.prefill(q, k, v, PSI[psi], n_psi=n_psi, prf_w=None if w is None else w[None], normalize=normalize,
                       eps=1e-3, log_gate=lg, S0=None if S0 is None else S0[None],
                       Z0=None if Z0 is None else Z0[None])[0]
    ref = brute.quadratic_gated(oracle.as_f64(q[0]), oracle.as_f64(k[0]), oracle.as_f64(v[0]), PSI[psi],
                                lg[0].double().numpy(), normalize, 1e-3, None if w is None else oracle.as_f64(w),
                                S0=S0, Z0=Z0)
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-11 * np.abs(ref).max())


def test_constant_gate_is_scalar_decay():
    """The same gate in every channel and at every token is the per-head decay gamma."""
    T, d = 60, 8
    q, k, v = _rand((2, T, d), 31, 0.5), _rand((2, T, d), 32, 0.5), _rand((2, T, d), 33)
    lg = torch.full((2, T, d), math.log(0.93), dtype=torch.float32)
    gam = math.exp(float(lg[0, 0, 0]))  # the decay the stored fp32 log gate stands for
    for normalize in (0, 1):
        a = oracle.prefill(q, k, v, oracle.PSI_ELU1, normalize=normalize, log_gate=lg)
        b = oracle.prefill(q, k, v, oracle.PSI_ELU1, normalize=normalize, gamma=[gam, gam])
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_zero_log_gate_is_no_decay():
    T, d = 40, 8
    q, k, v = _rand((1, T, d), 41, 0.5), _rand((1, T, d), 42, 0.5), _rand((1, T, d), 43)
    a = oracle.prefill(q, k, v, oracle.PSI_ELU1, log_gate=torch.zeros((1, T, d)))
    b = oracle.prefill(q, k, v, oracle.PSI_ELU1)
    assert np.array_equal(a, b)


def test_gated_decode_equals_prefill():
    T, d = 30, 8
    q, k, v = _rand((3, T, d), 51, 0.5), _rand((3, T, d), 52, 0.5), _rand((3, T, d), 53)
    lg = _gates((3, T, d), 54)
    ref = oracle.prefill(q, k, v, oracle.PSI_ELU1, log_gate=lg)
    S, Z = np.zeros((3, d, d)), np.zeros((3, d))
    for t in range(T):
        o = oracle.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(), S, Z,
                               oracle.PSI_ELU1, log_gate=lg[:, t].contiguous())
        assert np.array_equal(o, ref[:, t])


def test_strong_gate_forgets_the_past():
    """A gate of exp(-60) in every channel at token r wipes what came before (to e^-60):
    afterwards the outputs are those of the sequence that starts at r."""
    T, d, r = 50, 8, 20
    q, k, v = _rand((1, T, d), 61, 0.5), _rand((1, T, d), 62, 0.5), _rand((1, T, d), 63)
    lg = _gates((1, T, d), 64, lo=-1.0)
    lg[0, r] = -60.0
    full = oracle.prefill(q, k, v, oracle.PSI_ELU1, log_gate=lg)[0]
    tail = oracle.prefill(q[:, r:].contiguous(), k[:, r:].contiguous(), v[:, r:].contiguous(), oracle.PSI_ELU1,
                          log_gate=lg[:, r:].contiguous())[0]
    np.testing.assert_allclose(full[r:], tail, rtol=1e-20 + 1e-12, atol=1e-20)
