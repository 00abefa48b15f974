/*
 * linattn_oracle.c -- plain, slow fp64 CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes is the definition of causal linear attention, token by token,
 * in fp64 on the exact stored input values (bf16 or fp32, upcast exactly):
 *
 *   for t = 1..T:  f = psi(k_t);  S = gamma*S + f v_t^T;  Z = gamma*Z + f
 *                  g = psi(q_t);  o_t = g^T S / (g . Z + eps)   (or g^T S alone)
 *
 *  - the recurrent dual S_t = S_{t-1} + phi(k_t)^T v_t, z_t = z_{t-1} + phi(k_t)^T,
 *    o_t = phi(q_t) S_t / phi(q_t) z_t: "Linear Attention and Retentive Networks",
 *    section "The Recurrent Dual";
 *  - the decayed recurrence S_t = gamma S_{t-1} + k_t^T v_t, o_t = q_t S_t:
 *    same page, "Retentive Networks", recurrent representation (B);
 *  - eps added to the denominator dot product: "Log-Depth Chunked Linear-Attention
 *    Scan", Implementation notes (z_t = phi_q S / (phi_q Z + eps));
 *  - the normaliser Z decays with the same gamma as S, and every step updates the
 *    state before reading it (the inclusive sum over i <= t of the mathematical
 *    statement on the same page);
 *  - feature maps: identity; elu(x)+1 ("Linear Attention and Retentive Networks",
 *    "The Associative Property and Linear Kernel Formulation"); positive random
 *    features psi(x)_p = exp(w_p . x - |x|^2/2) / sqrt(m) ("Linearized 2-Simplicial
 *    Attention", section 3.2 and appendix "Feature scaling": the m^{-1/2} factor
 *    sits on each feature vector);
 *  - the same features with the log-space shift of the query row (same page,
 *    appendix B.2): psi(q)_p = exp(l_p - max_r l_r) / sqrt(m) with
 *    l_p = w_p . q - |q|^2/2, the shift depending on the query row only and shared by
 *    numerator and denominator; key features unshifted.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_PSI_IDENTITY = 0, ORC_PSI_ELU1 = 1, ORC_PSI_PRF = 2, ORC_PSI_PRF_QSHIFT = 3 };
#define ORC_IS_PRF(psi) ((psi) == ORC_PSI_PRF || (psi) == ORC_PSI_PRF_QSHIFT)
enum { ORC_BF16 = 0, ORC_F32 = 1 };

/* Exact upcast of one stored element. bf16 is the top half of an IEEE fp32. */
static double load_elem(const void* base, int dtype, size_t idx) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static void load_vec(const void* base, int dtype, size_t off, int n, double* out) {
  for (int j = 0; j < n; ++j) out[j] = load_elem(base, dtype, off + (size_t)j);
}

/* psi(x) for one vector x[d_k] -> out[n_psi]. w is the head's bank [n_psi][d_k] (PRF only). */
void oracle_feature_f64(int psi, int d_k, int n_psi, const double* x, const double* w, double* out) {
  if (psi == ORC_PSI_IDENTITY) {
    for (int j = 0; j < d_k; ++j) out[j] = x[j];
  } else if (psi == ORC_PSI_ELU1) {
    /* elu(x) = x for x > 0, exp(x) - 1 otherwise; plus one. */
    for (int j = 0; j < d_k; ++j) out[j] = x[j] > 0.0 ? x[j] + 1.0 : exp(x[j]);
  } else {
    /* log-features l_p = w_p . x - |x|^2/2; PRF_QSHIFT subtracts their maximum */
    double sq = 0.0;
    for (int j = 0; j < d_k; ++j) sq += x[j] * x[j];
    double inv_sqrt_m = 1.0 / sqrt((double)n_psi);
    for (int p = 0; p < n_psi; ++p) {
      double dot = 0.0;
      for (int j = 0; j < d_k; ++j) dot += w[(size_t)p * d_k + j] * x[j];
      out[p] = dot - 0.5 * sq;
    }
    double shift = 0.0;
    if (psi == ORC_PSI_PRF_QSHIFT) {
      shift = out[0];
      for (int p = 1; p < n_psi; ++p) shift = out[p] > shift ? out[p] : shift;
    }
    for (int p = 0; p < n_psi; ++p) out[p] = exp(out[p] - shift) * inv_sqrt_m;
  }
}

/* One token of the recurrence on the state (S[n_psi][d_v], Z[n_psi]).
 * k_t, v_t update the state; if q_t is given, o_t is written afterwards. */
static void recurrence_step(int psi, int d_k, int d_v, int n_psi, const double* w, double gamma,
                            int normalize, double eps, const double* kt, const double* vt,
                            const double* qt, double* S, double* Z, double* f, double* g,
                            double* ot) {
  /* keys never take the query-row shift */
  oracle_feature_f64(psi == ORC_PSI_PRF_QSHIFT ? ORC_PSI_PRF : psi, d_k, n_psi, kt, w, f);
  for (int p = 0; p < n_psi; ++p) {
    double* row = S + (size_t)p * d_v;
    for (int e = 0; e < d_v; ++e) row[e] = gamma * row[e] + f[p] * vt[e];
    if (Z) Z[p] = gamma * Z[p] + f[p];
  }
  if (!qt) return;
  oracle_feature_f64(psi, d_k, n_psi, qt, w, g);
  double den = 0.0;
  if (normalize) {
    for (int p = 0; p < n_psi; ++p) den += g[p] * Z[p];
    den += eps;
  }
  /* numerator g^T S, summed over p in increasing order for every column e */
  for (int e = 0; e < d_v; ++e) ot[e] = 0.0;
  for (int p = 0; p < n_psi; ++p) {
    const double* row = S + (size_t)p * d_v;
    for (int e = 0; e < d_v; ++e) ot[e] += g[p] * row[e];
  }
  if (normalize)
    for (int e = 0; e < d_v; ++e) ot[e] = ot[e] / den;
}

/*
 * Prefill oracle over nblk independent (batch, head) blocks, OpenMP across blocks.
 *   q, k: [nblk][T][d_k], v: [nblk][T][d_v], stored as in_dtype (q may be NULL: state only)
 *   w: PRF banks [H_w][n_psi][d_k] stored as in_dtype (NULL unless psi == PRF);
 *   w_head[b]: which bank block b uses (NULL => bank 0)
 *   gamma[b]: the decay of block b (fp32 value passed as double); NULL => 1
 *   S0, Z0: initial state [nblk][n_psi][d_v], [nblk][n_psi] (NULL => zero)
 *   o: [nblk][T][d_v] (NULL if q is NULL); S_out, Z_out: final state (NULL => not written)
 *   nthreads <= 0 => OpenMP default.
 * Returns 0, or -1 on an allocation failure or bad argument.
 */
int oracle_prefill_f64(int nblk, int T, int d_k, int d_v, int n_psi, int psi, int in_dtype,
                       const void* q, const void* k, const void* v, const void* w,
                       const int32_t* w_head, const double* gamma, int normalize, double eps,
                       const double* S0, const double* Z0, double* o, double* S_out,
                       double* Z_out, int nthreads) {
  if (nblk < 0 || T < 0 || d_k <= 0 || d_v <= 0 || n_psi <= 0) return -1;
  if (!ORC_IS_PRF(psi) && n_psi != d_k) return -1;
  if (ORC_IS_PRF(psi) && !w) return -1;
  if (q && !o) return -1;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
#endif
  for (int b = 0; b < nblk; ++b) {
    double* S = (double*)calloc((size_t)n_psi * d_v, sizeof(double));
    double* Z = (double*)calloc((size_t)n_psi, sizeof(double));
    double* f = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* g = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* kt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* qt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* vt = (double*)malloc(sizeof(double) * (size_t)d_v);
    double* wd = NULL;
    if (ORC_IS_PRF(psi)) wd = (double*)malloc(sizeof(double) * (size_t)n_psi * d_k);
    if (!S || !Z || !f || !g || !kt || !qt || !vt || (ORC_IS_PRF(psi) && !wd)) {
      err |= 1;
    } else {
      if (wd) {
        size_t hw = w_head ? (size_t)w_head[b] : 0;
        load_vec(w, in_dtype, hw * (size_t)n_psi * d_k, n_psi * d_k, wd);
      }
      if (S0) memcpy(S, S0 + (size_t)b * n_psi * d_v, sizeof(double) * (size_t)n_psi * d_v);
      if (Z0) memcpy(Z, Z0 + (size_t)b * n_psi, sizeof(double) * (size_t)n_psi);
      double gm = gamma ? gamma[b] : 1.0;
      for (int t = 0; t < T; ++t) {
        size_t rowk = ((size_t)b * T + t) * d_k, rowv = ((size_t)b * T + t) * d_v;
        load_vec(k, in_dtype, rowk, d_k, kt);
        load_vec(v, in_dtype, rowv, d_v, vt);
        if (q) load_vec(q, in_dtype, rowk, d_k, qt);
        recurrence_step(psi, d_k, d_v, n_psi, wd, gm, normalize, eps, kt, vt, q ? qt : NULL, S, Z,
                        f, g, q ? o + rowv : NULL);
      }
      if (S_out) memcpy(S_out + (size_t)b * n_psi * d_v, S, sizeof(double) * (size_t)n_psi * d_v);
      if (Z_out) memcpy(Z_out + (size_t)b * n_psi, Z, sizeof(double) * (size_t)n_psi);
    }
    free(S); free(Z); free(f); free(g); free(kt); free(qt); free(vt); free(wd);
  }
  return err ? -1 : 0;
}

/*
 * One decode step for nblk independent states, in place: the same loop body as
 * the prefill recurrence applied to a single token ("Linear Attention and
 * Retentive Networks", The Recurrent Dual: O(1) memory per step).
 *   q, k: [nblk][d_k], v: [nblk][d_v] (in_dtype); S [nblk][n_psi][d_v], Z [nblk][n_psi] (fp64, in/out;
 *   Z may be NULL when normalize == 0); o [nblk][d_v].
 */
int oracle_decode_step_f64(int nblk, int d_k, int d_v, int n_psi, int psi, int in_dtype,
                           const void* q, const void* k, const void* v, const void* w,
                           const int32_t* w_head, const double* gamma, int normalize, double eps,
                           double* S, double* Z, double* o, int nthreads) {
  if (nblk < 0 || d_k <= 0 || d_v <= 0 || n_psi <= 0 || !q || !k || !v || !S || !o) return -1;
  if (!ORC_IS_PRF(psi) && n_psi != d_k) return -1;
  if (ORC_IS_PRF(psi) && !w) return -1;
  if (normalize && !Z) return -1;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(| : err)
#endif
  for (int b = 0; b < nblk; ++b) {
    double* f = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* g = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* kt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* qt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* vt = (double*)malloc(sizeof(double) * (size_t)d_v);
    double* wd = NULL;
    if (ORC_IS_PRF(psi)) wd = (double*)malloc(sizeof(double) * (size_t)n_psi * d_k);
    if (!f || !g || !kt || !qt || !vt || (ORC_IS_PRF(psi) && !wd)) {
      err |= 1;
    } else {
      if (wd) {
        size_t hw = w_head ? (size_t)w_head[b] : 0;
        load_vec(w, in_dtype, hw * (size_t)n_psi * d_k, n_psi * d_k, wd);
      }
      load_vec(k, in_dtype, (size_t)b * d_k, d_k, kt);
      load_vec(q, in_dtype, (size_t)b * d_k, d_k, qt);
      load_vec(v, in_dtype, (size_t)b * d_v, d_v, vt);
      recurrence_step(psi, d_k, d_v, n_psi, wd, gamma ? gamma[b] : 1.0, normalize, eps, kt, vt, qt,
                      S + (size_t)b * n_psi * d_v, Z ? Z + (size_t)b * n_psi : NULL, f, g,
                      o + (size_t)b * d_v);
    }
    free(f); free(g); free(kt); free(qt); free(vt); free(wd);
  }
  return err ? -1 : 0;
}

/*
 * Gated recurrence ("Linear Attention and Retentive Networks", Data-Dependent Gating
 * Mechanism: S_t = G_t . S_{t-1} + k_t^T v_t with G_t = alpha_t 1^T, one forget gate per
 * state row, i.e. per key feature): for every token t,
 *   alpha = exp(log_gate_t)                                  (n_psi gates)
 *   S[p][:] = alpha[p] S[p][:] + psi(k_t)[p] v_t^T;  Z[p] = alpha[p] Z[p] + psi(k_t)[p]
 *   o_t = psi(q_t)^T S / (psi(q_t) . Z + eps)   (or the numerator alone)
 * log_gate: fp32 [nblk][T][n_psi] (fp32 values used exactly); other arguments as for
 * oracle_prefill_f64. Update first, then read, as in the ungated recurrence.
 */
static void gated_step(int psi, int d_k, int d_v, int n_psi, const double* w, const float* lg,
                       int normalize, double eps, const double* kt, const double* vt, const double* qt,
                       double* S, double* Z, double* f, double* g, double* ot) {
  oracle_feature_f64(psi == ORC_PSI_PRF_QSHIFT ? ORC_PSI_PRF : psi, d_k, n_psi, kt, w, f);
  for (int p = 0; p < n_psi; ++p) {
    const double alpha = exp((double)lg[p]);
    double* row = S + (size_t)p * d_v;
    for (int e = 0; e < d_v; ++e) row[e] = alpha * row[e] + f[p] * vt[e];
    if (Z) Z[p] = alpha * Z[p] + f[p];
  }
  if (!qt) return;
  oracle_feature_f64(psi, d_k, n_psi, qt, w, g);
  double den = 0.0;
  if (normalize) {
    for (int p = 0; p < n_psi; ++p) den += g[p] * Z[p];
    den += eps;
  }
  for (int e = 0; e < d_v; ++e) ot[e] = 0.0;
  for (int p = 0; p < n_psi; ++p) {
    const double* row = S + (size_t)p * d_v;
    for (int e = 0; e < d_v; ++e) ot[e] += g[p] * row[e];
  }
  if (normalize)
    for (int e = 0; e < d_v; ++e) ot[e] = ot[e] / den;
}

int oracle_prefill_gated_f64(int nblk, int T, int d_k, int d_v, int n_psi, int psi, int in_dtype,
                             const void* q, const void* k, const void* v, const void* w,
                             const int32_t* w_head, const float* log_gate, int normalize, double eps,
                             const double* S0, const double* Z0, double* o, double* S_out,
                             double* Z_out, int nthreads) {
  if (nblk < 0 || T < 0 || d_k <= 0 || d_v <= 0 || n_psi <= 0 || !log_gate) return -1;
  if (!ORC_IS_PRF(psi) && n_psi != d_k) return -1;
  if (ORC_IS_PRF(psi) && !w) return -1;
  if (q && !o) return -1;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
#endif
  for (int b = 0; b < nblk; ++b) {
    double* S = (double*)calloc((size_t)n_psi * d_v, sizeof(double));
    double* Z = (double*)calloc((size_t)n_psi, sizeof(double));
    double* f = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* g = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* kt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* qt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* vt = (double*)malloc(sizeof(double) * (size_t)d_v);
    double* wd = NULL;
    if (ORC_IS_PRF(psi)) wd = (double*)malloc(sizeof(double) * (size_t)n_psi * d_k);
    if (!S || !Z || !f || !g || !kt || !qt || !vt || (ORC_IS_PRF(psi) && !wd)) {
      err |= 1;
    } else {
      if (wd) {
        size_t hw = w_head ? (size_t)w_head[b] : 0;
        load_vec(w, in_dtype, hw * (size_t)n_psi * d_k, n_psi * d_k, wd);
      }
      if (S0) memcpy(S, S0 + (size_t)b * n_psi * d_v, sizeof(double) * (size_t)n_psi * d_v);
      if (Z0) memcpy(Z, Z0 + (size_t)b * n_psi, sizeof(double) * (size_t)n_psi);
      for (int t = 0; t < T; ++t) {
        size_t rowk = ((size_t)b * T + t) * d_k, rowv = ((size_t)b * T + t) * d_v;
        load_vec(k, in_dtype, rowk, d_k, kt);
        load_vec(v, in_dtype, rowv, d_v, vt);
        if (q) load_vec(q, in_dtype, rowk, d_k, qt);
        gated_step(psi, d_k, d_v, n_psi, wd, log_gate + ((size_t)b * T + t) * n_psi, normalize, eps, kt, vt,
                   q ? qt : NULL, S, Z, f, g, q ? o + rowv : NULL);
      }
      if (S_out) memcpy(S_out + (size_t)b * n_psi * d_v, S, sizeof(double) * (size_t)n_psi * d_v);
      if (Z_out) memcpy(Z_out + (size_t)b * n_psi, Z, sizeof(double) * (size_t)n_psi);
    }
    free(S); free(Z); free(f); free(g); free(kt); free(qt); free(vt); free(wd);
  }
  return err ? -1 : 0;
}

/* One gated decode step for nblk states in place (log_gate: fp32 [nblk][n_psi]). */
int oracle_decode_step_gated_f64(int nblk, int d_k, int d_v, int n_psi, int psi, int in_dtype,
                                 const void* q, const void* k, const void* v, const void* w,
                                 const int32_t* w_head, const float* log_gate, int normalize, double eps,
                                 double* S, double* Z, double* o, int nthreads) {
  if (nblk < 0 || d_k <= 0 || d_v <= 0 || n_psi <= 0 || !q || !k || !v || !S || !o || !log_gate) return -1;
  if (!ORC_IS_PRF(psi) && n_psi != d_k) return -1;
  if (ORC_IS_PRF(psi) && !w) return -1;
  if (normalize && !Z) return -1;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(| : err)
#endif
  for (int b = 0; b < nblk; ++b) {
    double* f = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* g = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* kt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* qt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* vt = (double*)malloc(sizeof(double) * (size_t)d_v);
    double* wd = NULL;
    if (ORC_IS_PRF(psi)) wd = (double*)malloc(sizeof(double) * (size_t)n_psi * d_k);
    if (!f || !g || !kt || !qt || !vt || (ORC_IS_PRF(psi) && !wd)) {
      err |= 1;
    } else {
      if (wd) {
        size_t hw = w_head ? (size_t)w_head[b] : 0;
        load_vec(w, in_dtype, hw * (size_t)n_psi * d_k, n_psi * d_k, wd);
      }
      load_vec(k, in_dtype, (size_t)b * d_k, d_k, kt);
      load_vec(q, in_dtype, (size_t)b * d_k, d_k, qt);
      load_vec(v, in_dtype, (size_t)b * d_v, d_v, vt);
      gated_step(psi, d_k, d_v, n_psi, wd, log_gate + (size_t)b * n_psi, normalize, eps, kt, vt, qt,
                 S + (size_t)b * n_psi * d_v, Z ? Z + (size_t)b * n_psi : NULL, f, g, o + (size_t)b * d_v);
    }
    free(f); free(g); free(kt); free(qt); free(vt); free(wd);
  }
  return err ? -1 : 0;
}

/*
 * Vector-Jacobian product of the feature map: dx = J_psi(x)^T dpsi for one vector x[d_k].
 *   identity: dx = dpsi
 *   elu+1:    dx_j = dpsi_j * (1 if x_j > 0 else exp(x_j))   (the derivative of elu, continuous at 0)
 *   PRF:      psi_p = exp(l_p) / sqrt(m), l_p = w_p . x - |x|^2/2, dl_p/dx = w_p - x, so
 *             dx = sum_p dpsi_p psi_p (w_p - x)
 *   PRF with the query-row shift: l_p - l_r* with r* the (first) largest l, so
 *             dx = sum_p dpsi_p psi_p (w_p - w_r*)   (the -x terms cancel with the shift's)
 * psi_buf: n_psi doubles of scratch.
 */
static void feature_vjp(int psi, int d_k, int n_psi, const double* x, const double* w, const double* dpsi,
                        double* dx, double* psi_buf) {
  if (psi == ORC_PSI_IDENTITY) {
    for (int j = 0; j < d_k; ++j) dx[j] = dpsi[j];
  } else if (psi == ORC_PSI_ELU1) {
    for (int j = 0; j < d_k; ++j) dx[j] = dpsi[j] * (x[j] > 0.0 ? 1.0 : exp(x[j]));
  } else {
    oracle_feature_f64(psi, d_k, n_psi, x, w, psi_buf);
    int rstar = -1;
    if (psi == ORC_PSI_PRF_QSHIFT) {
      /* argmax of w_r . x (the -|x|^2/2 term is common to every r) */
      double best = 0.0;
      for (int r = 0; r < n_psi; ++r) {
        double dot = 0.0;
        for (int j = 0; j < d_k; ++j) dot += w[(size_t)r * d_k + j] * x[j];
        if (r == 0 || dot > best) { best = dot; rstar = r; }
      }
    }
    for (int j = 0; j < d_k; ++j) dx[j] = 0.0;
    double c = 0.0; /* sum_p dpsi_p psi_p */
    for (int p = 0; p < n_psi; ++p) {
      const double a = dpsi[p] * psi_buf[p];
      c += a;
      for (int j = 0; j < d_k; ++j) dx[j] += a * w[(size_t)p * d_k + j];
    }
    for (int j = 0; j < d_k; ++j)
      dx[j] -= c * (rstar >= 0 ? w[(size_t)rstar * d_k + j] : x[j]);
  }
}

/*
 * Backward of the prefill recurrence of oracle_prefill_f64: the gradients of
 * L = sum_t dout_t . o_t with respect to q, k, v and the initial state. It is the adjoint of
 * the token loop, one sweep forward and one back ("Log-Depth Chunked Linear-Attention Scan",
 * Mathematical statement, for o_t as a read of the inclusive prefix state; the chain rule for
 * the rest):
 *   read at t (g_t = psi(q_t)): num_t = g_t^T S_t, den_t = g_t . Z_t + eps, o_t = num_t / den_t
 *     dnum_t = dout_t / den_t, dden_t = -(dout_t . o_t) / den_t   (normalize = 0: dnum = dout,
 *     dden = 0), and dg_t = S_t dnum_t + Z_t dden_t
 *   write at t (f_t = psi(k_t)): S_t = gamma S_{t-1} + f_t v_t^T, Z_t = gamma Z_{t-1} + f_t. The
 *     adjoint of S_t gathers every later read: R_t = gamma R_{t+1} + g_t dnum_t^T and
 *     RZ_t = gamma RZ_{t+1} + g_t dden_t, so df_t = R_t v_t + RZ_t and dv_t = R_t^T f_t
 *   initial state: dS0 = gamma R_0, dZ0 = gamma RZ_0
 * and dq_t, dk_t through feature_vjp (keys never take the query-row shift). gamma and the
 * PRF bank are constants (no gradient).
 *   dout: fp64 [nblk][T][d_v]; dq, dk: fp64 [nblk][T][d_k]; dv: fp64 [nblk][T][d_v];
 *   dS0, dZ0: fp64 [nblk][n_psi][d_v], [nblk][n_psi], or NULL (not written).
 * Other arguments as for oracle_prefill_f64.
 */
int oracle_prefill_backward_f64(int nblk, int T, int d_k, int d_v, int n_psi, int psi, int in_dtype,
                                const void* q, const void* k, const void* v, const void* w,
                                const int32_t* w_head, const double* gamma, int normalize, double eps,
                                const double* S0, const double* Z0, const double* dout, double* dq,
                                double* dk, double* dv, double* dS0, double* dZ0, int nthreads) {
  if (nblk < 0 || T < 0 || d_k <= 0 || d_v <= 0 || n_psi <= 0) return -1;
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (!ORC_IS_PRF(psi) && n_psi != d_k) return -1;
  if (ORC_IS_PRF(psi) && !w) return -1;
  const int psi_k = psi == ORC_PSI_PRF_QSHIFT ? ORC_PSI_PRF : psi;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
#endif
  for (int b = 0; b < nblk; ++b) {
    const size_t nS = (size_t)n_psi * d_v;
    double* S = (double*)calloc(nS, sizeof(double));
    double* Z = (double*)calloc((size_t)n_psi, sizeof(double));
    double* f = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* dg = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* buf = (double*)malloc(sizeof(double) * (size_t)n_psi);
    double* kt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* qt = (double*)malloc(sizeof(double) * (size_t)d_k);
    double* vt = (double*)malloc(sizeof(double) * (size_t)d_v);
    double* ot = (double*)malloc(sizeof(double) * (size_t)d_v);
    /* per-token records of the forward sweep for the reverse one: g_t, dnum_t, dden_t */
    double* G = (double*)malloc(sizeof(double) * ((size_t)T * n_psi + 1));
    double* DN = (double*)malloc(sizeof(double) * ((size_t)T * d_v + 1));
    double* DD = (double*)malloc(sizeof(double) * ((size_t)T + 1));
    double* wd = NULL;
    if (ORC_IS_PRF(psi)) wd = (double*)malloc(sizeof(double) * (size_t)n_psi * d_k);
    if (!S || !Z || !f || !dg || !buf || !kt || !qt || !vt || !ot || !G || !DN || !DD || (ORC_IS_PRF(psi) && !wd)) {
      err |= 1;
    } else {
      if (wd) {
        size_t hw = w_head ? (size_t)w_head[b] : 0;
        load_vec(w, in_dtype, hw * (size_t)n_psi * d_k, n_psi * d_k, wd);
      }
      if (S0) memcpy(S, S0 + (size_t)b * nS, sizeof(double) * nS);
      if (Z0) memcpy(Z, Z0 + (size_t)b * n_psi, sizeof(double) * (size_t)n_psi);
      const double gm = gamma ? gamma[b] : 1.0;
      /* forward sweep: states, outputs, dnum, dden, and dq */
      for (int t = 0; t < T; ++t) {
        const size_t rowk = ((size_t)b * T + t) * d_k, rowv = ((size_t)b * T + t) * d_v;
        load_vec(k, in_dtype, rowk, d_k, kt);
        load_vec(v, in_dtype, rowv, d_v, vt);
        load_vec(q, in_dtype, rowk, d_k, qt);
        oracle_feature_f64(psi_k, d_k, n_psi, kt, wd, f);
        for (int p = 0; p < n_psi; ++p) {
          double* row = S + (size_t)p * d_v;
          for (int e = 0; e < d_v; ++e) row[e] = gm * row[e] + f[p] * vt[e];
          Z[p] = gm * Z[p] + f[p];
        }
        double* g = G + (size_t)t * n_psi;
        oracle_feature_f64(psi, d_k, n_psi, qt, wd, g);
        for (int e = 0; e < d_v; ++e) ot[e] = 0.0;
        for (int p = 0; p < n_psi; ++p)
          for (int e = 0; e < d_v; ++e) ot[e] += g[p] * S[(size_t)p * d_v + e];
        const double* dot_ = dout + rowv;
        double* dn = DN + (size_t)t * d_v;
        double dden = 0.0;
        if (normalize) {
          double den = eps;
          for (int p = 0; p < n_psi; ++p) den += g[p] * Z[p];
          double a = 0.0;
          for (int e = 0; e < d_v; ++e) {
            ot[e] /= den;
            a += dot_[e] * ot[e];
            dn[e] = dot_[e] / den;
          }
          dden = -a / den;
        } else {
          for (int e = 0; e < d_v; ++e) dn[e] = dot_[e];
        }
        DD[t] = dden;
        for (int p = 0; p < n_psi; ++p) {
          double a = 0.0;
          for (int e = 0; e < d_v; ++e) a += S[(size_t)p * d_v + e] * dn[e];
          dg[p] = a + Z[p] * dden;
        }
        feature_vjp(psi, d_k, n_psi, qt, wd, dg, dq + rowk, buf);
      }
      /* reverse sweep: the adjoint state (R, RZ), dk and dv */
      memset(S, 0, sizeof(double) * nS);
      memset(Z, 0, sizeof(double) * (size_t)n_psi);
      double* R = S;
      double* RZ = Z;
      for (int t = T - 1; t >= 0; --t) {
        const size_t rowk = ((size_t)b * T + t) * d_k, rowv = ((size_t)b * T + t) * d_v;
        const double* g = G + (size_t)t * n_psi;
        const double* dn = DN + (size_t)t * d_v;
        for (int p = 0; p < n_psi; ++p) {
          double* row = R + (size_t)p * d_v;
          for (int e = 0; e < d_v; ++e) row[e] = gm * row[e] + g[p] * dn[e];
          RZ[p] = gm * RZ[p] + g[p] * DD[t];
        }
        load_vec(k, in_dtype, rowk, d_k, kt);
        load_vec(v, in_dtype, rowv, d_v, vt);
        oracle_feature_f64(psi_k, d_k, n_psi, kt, wd, f);
        for (int p = 0; p < n_psi; ++p) {
          double a = 0.0;
          for (int e = 0; e < d_v; ++e) a += R[(size_t)p * d_v + e] * vt[e];
          dg[p] = a + RZ[p];
        }
        for (int e = 0; e < d_v; ++e) {
          double a = 0.0;
          for (int p = 0; p < n_psi; ++p) a += R[(size_t)p * d_v + e] * f[p];
          dv[rowv + e] = a;
        }
        feature_vjp(psi_k, d_k, n_psi, kt, wd, dg, dk + rowk, buf);
      }
      if (dS0)
        for (size_t i = 0; i < nS; ++i) dS0[(size_t)b * nS + i] = gm * R[i];
      if (dZ0)
        for (int p = 0; p < n_psi; ++p) dZ0[(size_t)b * n_psi + p] = gm * RZ[p];
    }
    free(S); free(Z); free(f); free(dg); free(buf); free(kt); free(qt); free(vt); free(ot);
    free(G); free(DN); free(DD); free(wd);
  }
  return err ? -1 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
