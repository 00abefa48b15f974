"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle's C source, plants one mistake (a dropped term, a
wrong sign, index or scale, a transposed operand), builds the copy on the CPU and
runs the pin suite against it; the suite must fail. Nothing here touches a GPU or
the product library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linattn_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_backward_pins.py")]

MUTATIONS = {
    "S_not_decayed": [("row[e] = gamma * row[e] + f[p] * vt[e];", "row[e] = row[e] + f[p] * vt[e];")],
    "Z_not_decayed": [("if (Z) Z[p] = gamma * Z[p] + f[p];", "if (Z) Z[p] = Z[p] + f[p];")],
    "value_index_dropped": [("row[e] = gamma * row[e] + f[p] * vt[e];", "row[e] = gamma * row[e] + f[p] * vt[0];")],
    "eps_outside_ratio": [("    den += eps;\n", ""), ("ot[e] = ot[e] / den;", "ot[e] = ot[e] / den + eps;")],
    "eps_sign": [("den += eps;", "den -= eps;")],
    "elu_missing_plus_one": [("x[j] > 0.0 ? x[j] + 1.0 : exp(x[j])", "x[j] > 0.0 ? x[j] : exp(x[j])")],
    "elu_wrong_branch": [("x[j] > 0.0 ? x[j] + 1.0 : exp(x[j])", "x[j] > 0.0 ? exp(x[j]) : x[j] + 1.0")],
    "prf_norm_not_halved": [("out[p] = dot - 0.5 * sq;", "out[p] = dot - sq;")],
    "prf_norm_sign": [("out[p] = dot - 0.5 * sq;", "out[p] = dot + 0.5 * sq;")],
    "qshift_on_keys_too": [("oracle_feature_f64(psi == ORC_PSI_PRF_QSHIFT ? ORC_PSI_PRF : psi, d_k, n_psi, kt, w, f);",
                            "oracle_feature_f64(psi, d_k, n_psi, kt, w, f);")],
    "qshift_missing": [("if (psi == ORC_PSI_PRF_QSHIFT) {", "if (0) {")],
    "gate_after_write": [("for (int e = 0; e < d_v; ++e) row[e] = alpha * row[e] + f[p] * vt[e];",
                          "for (int e = 0; e < d_v; ++e) row[e] = alpha * (row[e] + f[p] * vt[e]);")],
    "gate_not_on_Z": [("if (Z) Z[p] = alpha * Z[p] + f[p];", "if (Z) Z[p] = Z[p] + f[p];")],
    "gate_of_previous_token": [("log_gate + ((size_t)b * T + t) * n_psi,",
                                "log_gate + ((size_t)b * T + (t > 0 ? t - 1 : 0)) * n_psi,")],
    "gate_exp_sign": [("const double alpha = exp((double)lg[p]);", "const double alpha = exp(-(double)lg[p]);")],
    "gate_channel_reversed": [("const double alpha = exp((double)lg[p]);",
                               "const double alpha = exp((double)lg[n_psi - 1 - p]);")],
    "qshift_min_not_max": [("shift = out[p] > shift ? out[p] : shift;", "shift = out[p] < shift ? out[p] : shift;")],
    "prf_scale_1_over_m": [("1.0 / sqrt((double)n_psi)", "1.0 / (double)n_psi")],
    "state_transposed": [("ot[e] += g[p] * row[e];",
                          "ot[e] += g[p] * S[(size_t)(e % n_psi) * d_v + (size_t)(p % d_v)];")],
    "gamma_of_block0": [("double gm = gamma ? gamma[b] : 1.0;", "double gm = gamma ? gamma[0] : 1.0;")],
    "bank_of_head0": [("size_t hw = w_head ? (size_t)w_head[b] : 0;\n        load_vec(w, in_dtype, hw",
                       "size_t hw = 0;\n        load_vec(w, in_dtype, hw")],
    "initial_Z_ignored": [("if (Z0) memcpy(Z, Z0", "if (0) memcpy(Z, Z0")],
    "query_feature_from_key": [("oracle_feature_f64(psi, d_k, n_psi, qt, w, g);",
                                "oracle_feature_f64(psi, d_k, n_psi, kt, w, g);")],
    # backward
    "bwd_dden_sign": [("dden = -a / den;", "dden = a / den;")],
    "bwd_dnum_not_scaled": [("dn[e] = dot_[e] / den;", "dn[e] = dot_[e];")],
    "bwd_adjoint_not_decayed": [("row[e] = gm * row[e] + g[p] * dn[e];", "row[e] = row[e] + g[p] * dn[e];")],
    "bwd_adjoint_Z_dropped": [("dg[p] = a + RZ[p];", "dg[p] = a;")],
    "bwd_dS0_missing_gamma": [("dS0[(size_t)b * nS + i] = gm * R[i];", "dS0[(size_t)b * nS + i] = R[i];")],
    "bwd_dv_from_query_feature": [("a += R[(size_t)p * d_v + e] * f[p];", "a += R[(size_t)p * d_v + e] * g[p];")],
    "bwd_dq_state_without_Z": [("dg[p] = a + Z[p] * dden;", "dg[p] = a;")],
    "bwd_elu_derivative_branch": [("dx[j] = dpsi[j] * (x[j] > 0.0 ? 1.0 : exp(x[j]));",
                                   "dx[j] = dpsi[j] * (x[j] > 0.0 ? exp(x[j]) : 1.0);")],
    "bwd_prf_norm_term_dropped": [("dx[j] -= c * (rstar >= 0 ? w[(size_t)rstar * d_k + j] : x[j]);",
                                   "dx[j] -= c * (rstar >= 0 ? w[(size_t)rstar * d_k + j] : 0.0);")],
    "bwd_qshift_argmax_ignored": [("if (psi == ORC_PSI_PRF_QSHIFT) {\n      /* argmax", "if (0) {\n      /* argmax")],
    "bwd_keys_take_the_shift": [("feature_vjp(psi_k, d_k, n_psi, kt, wd, dg, dk + rowk, buf);",
                                 "feature_vjp(psi, d_k, n_psi, kt, wd, dg, dk + rowk, buf);")],
    "bwd_adjoint_read_before_write": [
        ("        load_vec(k, in_dtype, rowk, d_k, kt);\n        load_vec(v, in_dtype, rowv, d_v, vt);\n        oracle_feature_f64(psi_k, d_k, n_psi, kt, wd, f);\n        for (int p = 0; p < n_psi; ++p) {\n          double a = 0.0;\n          for (int e = 0; e < d_v; ++e) a += R[(size_t)p * d_v + e] * vt[e];",
         "        load_vec(k, in_dtype, rowk, d_k, kt);\n        load_vec(v, in_dtype, rowv, d_v, vt);\n        oracle_feature_f64(psi_k, d_k, n_psi, kt, wd, f);\n        for (int p = 0; p < n_psi; ++p) {\n          double a = 0.0;\n          for (int e = 0; e < d_v; ++e) a += (R[(size_t)p * d_v + e] - g[p] * dn[e]) * vt[e];")],
}


def _run_mutation(name, edits, workdir):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"{name}: pattern not found: {old!r}"
        src = src.replace(old, new, 1)
    d = os.path.join(workdir, name)
    os.makedirs(d)
    c_path = os.path.join(d, "m.c")
    so_path = os.path.join(d, "m.so")
    open(c_path, "w").write(src)
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", c_path,
                    "-o", so_path, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, LINATTN_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode, r.stdout[-400:]


def test_pins_catch_every_planted_mistake():
    workdir = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda kv: _run_mutation(kv[0], kv[1], workdir), MUTATIONS.items()))
    finally:
        shutil.rmtree(workdir, ignore_errors=True)
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutations not caught by the pins: {survivors}"
    # a failure must be a failed assertion, not a broken harness (pytest exit code 1)
    odd = [(n, rc) for n, rc, _ in results if rc != 1]
    assert not odd, f"unexpected pytest exit codes: {odd}"


def test_unmutated_copy_passes():
    """Control: the same harness with an unmodified copy passes, so failures above are the planted mistakes."""
    workdir = tempfile.mkdtemp(prefix="oracle_ctl_")
    try:
        name, rc, out = _run_mutation("control", [], workdir)
    finally:
        shutil.rmtree(workdir, ignore_errors=True)
    assert rc == 0, out
