/*
 * msm_oracle.c -- plain, slow fp64 CPU oracle for the Momentum-Mamba selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call this file:
 * only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.  It shares no
 * code, header, table or constant with the HIP library.
 *
 * What it computes (all in double precision, inputs widened exactly from their stored dtype):
 *
 *   Momentum Mamba README, "Momentum Mamba Recurrence": per batch row b, channel d, state n
 *     v_t = beta * v_{t-1} + alpha * (delta_t * B_t * x_t)
 *     h_t = exp(delta_t * A) * h_{t-1} + v_t
 *     y_t = C_t . h_t                 (sum over the N states)
 *   with v and h starting at zero (the README states this for v; h is read the same way), or
 *   at a given initial state (h0, v0) -- the state a previous segment of the same sequence
 *   ended in (the README's `last_state` outputs, fed back to continue the scan).
 *   Layout of the arrays follows the selection semantics of "Mamba: Choosing What to Remember
 *   Based on the Input" (section "From input features to update coefficients"): B_t and C_t
 *   hold N values per position shared across channels, delta one value per channel, A fixed
 *   per (channel, state).  Row-major shapes:
 *     x, delta, y, dy, dx, ddelta : (Bt, L, D)
 *     A, dA                       : (D, N)
 *     B, C, dB, dC                : (Bt, L, N)
 *     Dskip, dDskip               : (D,)          (the per-channel skip weight of the Mamba block)
 *     last_h, last_v, h0, v0      : (Bt, D, N)
 *     dlast_h, dlast_v, dh0, dv0  : (Bt, D, N)
 *   The optional skip adds Dskip[d] * x to y ("Where the state computation sits in a Mamba
 *   block": a learned per-channel weight times the current input).  alpha does not scale it.
 *
 *   Backward (Momentum Mamba README, "Gradient Flow" and "Gradient Formulas"), for the loss
 *   l = sum(dy * y), read as follows (the page's listing reuses one variable for two adjoints):
 *     gh_t = C_t * dy_t + a_{t+1} * gh_{t+1}          adjoint of h_t
 *     gv_t = gh_t + beta * gv_{t+1}                   adjoint of v_t (v_t also feeds h_t)
 *     dx_t     += alpha * delta_t * B_t * gv_t
 *     ddelta_t += alpha * B_t * x_t * gv_t + A * a_t * h_{t-1} * gh_t
 *     dA       += delta_t * a_t * h_{t-1} * gh_t      (summed over b and t)
 *     dB_t     += alpha * delta_t * x_t * gv_t        (summed over channels d)
 *     dC_t     += dy_t * h_t                          (summed over channels d; from y = C.h)
 *     dx       += Dskip * dy,  dDskip = sum_{b,t} dy * x      (only when Dskip is given)
 *   The page writes the velocity adjoint as a pure beta-decay; the velocity also enters h_t
 *   directly, so its adjoint carries gh_t as well (checked by finite differences in tests).
 *   With terminal adjoints (the loss also holds <dlast_h, h_{L-1}> + <dlast_v, v_{L-1}>) they
 *   enter at the last step: gh_{L-1} gets dlast_h and gv_{L-1} gets dlast_v.  The adjoints of
 *   the initial state follow from h_0 = a_0 h0 + v_0 and v_0 = beta v0 + w_0:
 *     dh0 = a_0 * gh_0,   dv0 = beta * gv_0.
 *
 * The fused op (the selective-scan function of the Momentum Mamba README, "Low-Level
 * Functions", with its z, delta_bias and delta_softplus arguments; the block layout of "Where the
 * state computation sits in a Mamba block") wraps the same recurrence in two elementwise steps,
 * read as follows:
 *   delta_eff = softplus(delta + delta_bias[d])  with softplus(u) = log(1 + e^u), when
 *               delta_softplus is set; delta + delta_bias[d] otherwise (a NULL bias is zero);
 *   the scan above runs on delta_eff, giving y_raw (skip term included);
 *   y = y_raw * silu(z)  with silu(z) = z / (1 + e^{-z}), when a gate z (Bt, L, D) is given.
 * Its backward is the chain rule around the scan's backward:
 *   dy_eff = dy * silu(z),  dz = dy * y_raw * silu'(z),  silu'(z) = s (1 + z (1 - s)),
 *   s = 1 / (1 + e^{-z});   ddelta = ddelta_eff * s(delta + delta_bias) with softplus (the
 *   derivative of softplus is the logistic function), ddelta_eff without;
 *   ddelta_bias[d] = sum over b and t of ddelta.
 *
 * Zero-order hold (the fused op's `zoh` switch): the write coefficient delta of the first-order
 * form becomes g = (exp(delta A) - 1) / A, the exact discretisation Bbar = (Abar - 1) A^{-1} B of
 * the glossary page and of the complextorch page ("The diagonal SSM"), with g = delta at A = 0:
 *     v_t = beta v_{t-1} + alpha g_t B_t x_t.
 * Its derivatives: dg/ddelta = exp(delta A) = a and dg/dA = (delta a - g) / A, which is
 * delta^2 (1/2 + u/3 + u^2/8 + u^3/30 + ...) with u = delta A (used for |u| < 1e-3).  The
 * backward then reads dx += alpha g B gv, ddelta += alpha B x gv a + A a h gh,
 * dA += delta a h gh + alpha B x gv dg/dA, dB += alpha g x gv.
 *
 * Complex-valued SSM (Momentum Mamba README, "Complex Number Support": A, B and C complex; the
 * complextorch page, "The diagonal SSM": a complex diagonal state).  Per (b, d, n), with complex
 * a_t = exp(delta_t A), v_t = beta v_{t-1} + alpha delta_t B_t x_t, h_t = a_t h_{t-1} + v_t, and
 * the real output y_t = Re(sum_n C_t h_t) (+ Dskip x_t) -- x, delta, y stay real; the pages do not
 * say how a real output is taken from the complex readout, and the real part is the plainest
 * reading.  Complex arrays are interleaved (re, im): A (D, N, 2), B, C (Bt, L, N, 2), states
 * (Bt, D, N, 2).  Its backward, for the real loss sum(dy y) (+ <dlast_h, last_h> + <dlast_v,
 * last_v> over real and imaginary parts), with every complex gradient written as
 * G = dl/d(re) + i dl/d(im):
 *   gh_t = dy_t conj(C_t) + conj(a_{t+1}) gh_{t+1},   gv_t = gh_t + beta gv_{t+1}
 *   dx += alpha delta Re(conj(gv) B),   ddelta += alpha x Re(conj(gv) B) + Re(conj(gh) A a h_{t-1})
 *   dA += conj(delta a h_{t-1}) gh,     dB += alpha delta x gv,     dC += dy conj(h_t)
 *   dh0 = conj(a_0) gh_0,   dv0 = beta gv_0.
 *
 * Threads: the forward is split over (b, d) channel pairs, which are independent.  The
 * backward is split over batch rows b; dA and dDskip are first summed per row and the rows are
 * then added in order, so results do not depend on the thread count.
 */
#include <complex.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int msm_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Write coefficient of the update: delta (first-order) or (exp(delta A) - 1) / A (zero-order
 * hold, delta at A = 0), and its derivatives with respect to delta and A. */
static double write_coef(double dt, double An, int zoh) {
  if (!zoh) return dt;
  return An == 0.0 ? dt : expm1(dt * An) / An;
}

static double write_coef_ddelta(double dt, double An, int zoh) {
  return zoh ? exp(dt * An) : 1.0;
}

static double write_coef_dA(double dt, double An, int zoh) {
  if (!zoh) return 0.0;
  double u = dt * An;
  if (fabs(u) < 1e-3) return dt * dt * (0.5 + u / 3.0 + u * u / 8.0 + u * u * u / 30.0);
  return (dt * exp(u) - expm1(u) / An) / An;
}

static int fwd_core(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* Dskip, const double* h0, const double* v0,
                    double beta, double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N,
                    double* y, double* last_h, double* last_v, int zoh, int nthreads);
static int bwd_core(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* Dskip, const double* dy, const double* h0,
                    const double* v0, const double* dlast_h, const double* dlast_v, double beta,
                    double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N, double* dx,
                    double* ddelta, double* dA, double* dB, double* dC, double* dDskip,
                    double* dh0, double* dv0, int zoh, int nthreads);

/* Momentum recurrence, forward.  last_h / last_v, h0 / v0 and Dskip may be NULL (a NULL
 * initial state is zero). */
int msm_oracle_fwd(const double* x, const double* delta, const double* A, const double* B,
                   const double* C, const double* Dskip, const double* h0, const double* v0,
                   double beta, double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N,
                   double* y, double* last_h, double* last_v, int nthreads) {
  return fwd_core(x, delta, A, B, C, Dskip, h0, v0, beta, alpha, Bt, L, D, N, y, last_h, last_v,
                  0, nthreads);
}

static int fwd_core(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* Dskip, const double* h0, const double* v0,
                    double beta, double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N,
                    double* y, double* last_h, double* last_v, int zoh, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  set_threads(nthreads);
  int64_t nchan = Bt * D;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t bd = 0; bd < nchan; ++bd) {
    int64_t b = bd / D, d = bd % D;
    for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double v = v0 ? v0[(b * D + d) * N + n] : 0.0;
      double h = h0 ? h0[(b * D + d) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        double dt = delta[(b * L + t) * D + d];
        double xt = x[(b * L + t) * D + d];
        double a = exp(dt * A[d * N + n]);
        double g = write_coef(dt, A[d * N + n], zoh);
        double w = alpha * (g * B[(b * L + t) * N + n] * xt);
        v = beta * v + w;
        h = a * h + v;
        y[(b * L + t) * D + d] += C[(b * L + t) * N + n] * h;
      }
      if (last_h) last_h[(b * D + d) * N + n] = h;
      if (last_v) last_v[(b * D + d) * N + n] = v;
    }
    if (Dskip)
      for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] += Dskip[d] * x[(b * L + t) * D + d];
  }
  return 0;
}

/* Standard Mamba recurrence without a velocity state (Momentum Mamba README, "Standard Mamba
 * Recurrence"): h_t = exp(delta_t A) h_{t-1} + delta_t B_t x_t, y_t = C_t . h_t.
 * Kept separate from the momentum loop on purpose: the tests check that beta = 0, alpha = 1
 * of the momentum recurrence reproduces it. */
int msm_oracle_fwd_plain(const double* x, const double* delta, const double* A, const double* B,
                         const double* C, const double* Dskip, int64_t Bt, int64_t L, int64_t D,
                         int64_t N, double* y, double* last_h, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  set_threads(nthreads);
  int64_t nchan = Bt * D;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t bd = 0; bd < nchan; ++bd) {
    int64_t b = bd / D, d = bd % D;
    for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      double h = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        double dt = delta[(b * L + t) * D + d];
        double xt = x[(b * L + t) * D + d];
        h = exp(dt * A[d * N + n]) * h + dt * B[(b * L + t) * N + n] * xt;
        y[(b * L + t) * D + d] += C[(b * L + t) * N + n] * h;
      }
      if (last_h) last_h[(b * D + d) * N + n] = h;
    }
    if (Dskip)
      for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] += Dskip[d] * x[(b * L + t) * D + d];
  }
  return 0;
}

/* Backward of l = sum(dy * y) (+ <dlast_h, h_{L-1}> + <dlast_v, v_{L-1}>) for the momentum
 * recurrence started at (h0, v0).  All outputs are overwritten.  dDskip must be non-NULL when
 * Dskip is non-NULL and is ignored otherwise.  h0, v0, dlast_h, dlast_v may be NULL (zero);
 * dh0, dv0 may be NULL (not written). */
int msm_oracle_bwd(const double* x, const double* delta, const double* A, const double* B,
                   const double* C, const double* Dskip, const double* dy, const double* h0,
                   const double* v0, const double* dlast_h, const double* dlast_v, double beta,
                   double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N, double* dx,
                   double* ddelta, double* dA, double* dB, double* dC, double* dDskip,
                   double* dh0, double* dv0, int nthreads) {
  return bwd_core(x, delta, A, B, C, Dskip, dy, h0, v0, dlast_h, dlast_v, beta, alpha, Bt, L, D,
                  N, dx, ddelta, dA, dB, dC, dDskip, dh0, dv0, 0, nthreads);
}

static int bwd_core(const double* x, const double* delta, const double* A, const double* B,
                    const double* C, const double* Dskip, const double* dy, const double* h0,
                    const double* v0, const double* dlast_h, const double* dlast_v, double beta,
                    double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N, double* dx,
                    double* ddelta, double* dA, double* dB, double* dC, double* dDskip,
                    double* dh0, double* dv0, int zoh, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  if (Dskip && !dDskip) return 1;
  set_threads(nthreads);
  memset(dx, 0, sizeof(double) * (size_t)(Bt * L * D));
  memset(ddelta, 0, sizeof(double) * (size_t)(Bt * L * D));
  memset(dB, 0, sizeof(double) * (size_t)(Bt * L * N));
  memset(dC, 0, sizeof(double) * (size_t)(Bt * L * N));
  /* per-batch-row partial sums for the parameters shared across b */
  double* dA_rows = (double*)calloc((size_t)(Bt * D * N) + 1, sizeof(double));
  double* dD_rows = (double*)calloc((size_t)(Bt * D) + 1, sizeof(double));
  if (!dA_rows || !dD_rows) { free(dA_rows); free(dD_rows); return 2; }
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < Bt; ++b) {
    double* hs = (double*)malloc(sizeof(double) * (size_t)(L + 1));
    if (!hs) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t n = 0; n < N; ++n) {
        double An = A[d * N + n];
        /* forward, keeping every h_t: hs[t+1] = h_t, hs[0] = h_{-1} (the initial state) */
        const int64_t s_i = (b * D + d) * N + n;
        double v = v0 ? v0[s_i] : 0.0;
        double h = h0 ? h0[s_i] : 0.0;
        hs[0] = h;
        for (int64_t t = 0; t < L; ++t) {
          double dt = delta[(b * L + t) * D + d];
          double xt = x[(b * L + t) * D + d];
          double a = exp(dt * An);
          double g = write_coef(dt, An, zoh);
          v = beta * v + alpha * (g * B[(b * L + t) * N + n] * xt);
          h = a * h + v;
          hs[t + 1] = h;
        }
        /* reverse sweep; the terminal adjoint of h enters as a_next * gh_next at t = L-1 */
        double gh_next = dlast_h ? dlast_h[s_i] : 0.0, gv_next = 0.0, a_next = 1.0;
        for (int64_t t = L - 1; t >= 0; --t) {
          int64_t i = (b * L + t) * D + d;
          int64_t j = (b * L + t) * N + n;
          double dt = delta[i], xt = x[i], dyt = dy[i];
          double a = exp(dt * An);
          double gh = C[j] * dyt + a_next * gh_next;
          double gv = gh + beta * gv_next;
          if (t == L - 1 && dlast_v) gv += dlast_v[s_i];
          double hprev = hs[t]; /* h_{t-1} */
          double g = write_coef(dt, An, zoh);
          double gd = write_coef_ddelta(dt, An, zoh), gA = write_coef_dA(dt, An, zoh);
          dx[i] += alpha * g * B[j] * gv;
          ddelta[i] += alpha * B[j] * xt * gv * gd + An * a * hprev * gh;
          dA_rows[(b * D + d) * N + n] += dt * a * hprev * gh + alpha * B[j] * xt * gv * gA;
          dB[j] += alpha * g * xt * gv;
          dC[j] += dyt * hs[t + 1];
          gh_next = gh;
          gv_next = gv;
          a_next = a;
        }
        /* adjoints of the initial state (with L = 0 they are the terminal adjoints) */
        if (dh0) dh0[s_i] = L > 0 ? a_next * gh_next : (dlast_h ? dlast_h[s_i] : 0.0);
        if (dv0) dv0[s_i] = L > 0 ? beta * gv_next : (dlast_v ? dlast_v[s_i] : 0.0);
      }
      if (Dskip) {
        for (int64_t t = 0; t < L; ++t) {
          int64_t i = (b * L + t) * D + d;
          dx[i] += Dskip[d] * dy[i];
          dD_rows[b * D + d] += dy[i] * x[i];
        }
      }
    }
    free(hs);
  }
  if (failed) { free(dA_rows); free(dD_rows); return 2; }
  for (int64_t k = 0; k < D * N; ++k) {
    double s = 0.0;
    for (int64_t b = 0; b < Bt; ++b) s += dA_rows[b * D * N + k];
    dA[k] = s;
  }
  if (Dskip) {
    for (int64_t d = 0; d < D; ++d) {
      double s = 0.0;
      for (int64_t b = 0; b < Bt; ++b) s += dD_rows[b * D + d];
      dDskip[d] = s;
    }
  }
  free(dA_rows);
  free(dD_rows);
  return 0;
}

/* ---- the fused op: delta bias and softplus before the scan, the SiLU gate after it ---- */

static double softplus(double u) {
  /* log(1 + e^u), written so that neither branch overflows */
  return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u));
}

static double logistic(double u) {
  return u >= 0.0 ? 1.0 / (1.0 + exp(-u)) : exp(u) / (1.0 + exp(u));
}

static double silu(double z) { return z * logistic(z); }

static double silu_grad(double z) {
  double s = logistic(z);
  return s * (1.0 + z * (1.0 - s));
}

/* delta_eff as the fused op feeds it to the scan (see the header). */
static void effective_delta(const double* delta, const double* delta_bias, int delta_softplus,
                            int64_t Bt, int64_t L, int64_t D, double* out) {
  for (int64_t i = 0; i < Bt * L * D; ++i) {
    double u = delta[i] + (delta_bias ? delta_bias[i % D] : 0.0);
    out[i] = delta_softplus ? softplus(u) : u;
  }
}

/* Fused forward.  z, delta_bias, Dskip, h0, v0, y_raw (the output before the gate), last_h and
 * last_v may be NULL. */
int msm_oracle_fused_fwd(const double* x, const double* delta, const double* A, const double* B,
                         const double* C, const double* Dskip, const double* z,
                         const double* delta_bias, int delta_softplus, int zoh, const double* h0,
                         const double* v0, double beta, double alpha, int64_t Bt, int64_t L,
                         int64_t D, int64_t N, double* y, double* y_raw, double* last_h,
                         double* last_v, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  const size_t nxd = (size_t)(Bt * L * D);
  double* de = (double*)malloc(sizeof(double) * nxd + 1);
  double* yr = (double*)malloc(sizeof(double) * nxd + 1);
  if (!de || !yr) { free(de); free(yr); return 2; }
  effective_delta(delta, delta_bias, delta_softplus, Bt, L, D, de);
  int rc = fwd_core(x, de, A, B, C, Dskip, h0, v0, beta, alpha, Bt, L, D, N, yr, last_h, last_v,
                    zoh, nthreads);
  if (rc == 0) {
    for (size_t i = 0; i < nxd; ++i) {
      if (y_raw) y_raw[i] = yr[i];
      y[i] = z ? yr[i] * silu(z[i]) : yr[i];
    }
  }
  free(de);
  free(yr);
  return rc;
}

/* Fused backward: gradients of sum(dy * y) (+ the terminal-adjoint terms) with respect to the
 * fused op's inputs.  ddelta is the gradient of the raw delta (before bias and softplus).  dz
 * is required when z is given, ddelta_bias when delta_bias is given. */
int msm_oracle_fused_bwd(const double* x, const double* delta, const double* A, const double* B,
                         const double* C, const double* Dskip, const double* z,
                         const double* delta_bias, int delta_softplus, int zoh, const double* dy,
                         const double* h0, const double* v0, const double* dlast_h,
                         const double* dlast_v, double beta, double alpha, int64_t Bt, int64_t L,
                         int64_t D, int64_t N, double* dx, double* ddelta, double* dA,
                         double* dB, double* dC, double* dDskip, double* dz,
                         double* ddelta_bias, double* dh0, double* dv0, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  if ((z && !dz) || (delta_bias && !ddelta_bias)) return 1;
  const size_t nxd = (size_t)(Bt * L * D);
  double* de = (double*)malloc(sizeof(double) * nxd + 1);
  double* ge = (double*)malloc(sizeof(double) * nxd + 1);
  double* yr = (double*)malloc(sizeof(double) * nxd + 1);
  if (!de || !ge || !yr) { free(de); free(ge); free(yr); return 2; }
  effective_delta(delta, delta_bias, delta_softplus, Bt, L, D, de);
  int rc = 0;
  if (z) {
    /* the gate's backward needs the output before the gate */
    rc = fwd_core(x, de, A, B, C, Dskip, h0, v0, beta, alpha, Bt, L, D, N, yr, NULL, NULL, zoh,
                  nthreads);
    for (size_t i = 0; rc == 0 && i < nxd; ++i) {
      ge[i] = dy[i] * silu(z[i]);
      dz[i] = dy[i] * yr[i] * silu_grad(z[i]);
    }
  } else {
    memcpy(ge, dy, sizeof(double) * nxd);
  }
  if (rc == 0)
    rc = bwd_core(x, de, A, B, C, Dskip, ge, h0, v0, dlast_h, dlast_v, beta, alpha, Bt, L, D, N,
                  dx, ddelta, dA, dB, dC, dDskip, dh0, dv0, zoh, nthreads);
  if (rc == 0) {
    if (delta_softplus)
      for (size_t i = 0; i < nxd; ++i)
        ddelta[i] *= logistic(delta[i] + (delta_bias ? delta_bias[i % D] : 0.0));
    if (delta_bias) {
      for (int64_t d = 0; d < D; ++d) ddelta_bias[d] = 0.0;
      for (int64_t b = 0; b < Bt; ++b)
        for (int64_t t = 0; t < L; ++t)
          for (int64_t d = 0; d < D; ++d) ddelta_bias[d] += ddelta[(b * L + t) * D + d];
    }
  }
  free(de);
  free(ge);
  free(yr);
  return rc;
}

/* ---- complex-valued SSM (see the header) ---- */

static double complex cget(const double* p, int64_t i) { return p[2 * i] + I * p[2 * i + 1]; }

static void cput(double* p, int64_t i, double complex z) {
  p[2 * i] = creal(z);
  p[2 * i + 1] = cimag(z);
}

int msm_oracle_complex_fwd(const double* x, const double* delta, const double* A,
                           const double* B, const double* C, const double* Dskip,
                           const double* h0, const double* v0, double beta, double alpha,
                           int64_t Bt, int64_t L, int64_t D, int64_t N, double* y,
                           double* last_h, double* last_v, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  set_threads(nthreads);
  int64_t nchan = Bt * D;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t bd = 0; bd < nchan; ++bd) {
    int64_t b = bd / D, d = bd % D;
    for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const int64_t s_i = (b * D + d) * N + n;
      double complex v = v0 ? cget(v0, s_i) : 0.0;
      double complex h = h0 ? cget(h0, s_i) : 0.0;
      double complex An = cget(A, d * N + n);
      for (int64_t t = 0; t < L; ++t) {
        double dt = delta[(b * L + t) * D + d];
        double xt = x[(b * L + t) * D + d];
        double complex a = cexp(dt * An);
        double complex w = alpha * dt * xt * cget(B, (b * L + t) * N + n);
        v = beta * v + w;
        h = a * h + v;
        y[(b * L + t) * D + d] += creal(cget(C, (b * L + t) * N + n) * h);
      }
      if (last_h) cput(last_h, s_i, h);
      if (last_v) cput(last_v, s_i, v);
    }
    if (Dskip)
      for (int64_t t = 0; t < L; ++t) y[(b * L + t) * D + d] += Dskip[d] * x[(b * L + t) * D + d];
  }
  return 0;
}

int msm_oracle_complex_bwd(const double* x, const double* delta, const double* A,
                           const double* B, const double* C, const double* Dskip,
                           const double* dy, const double* h0, const double* v0,
                           const double* dlast_h, const double* dlast_v, double beta,
                           double alpha, int64_t Bt, int64_t L, int64_t D, int64_t N, double* dx,
                           double* ddelta, double* dA, double* dB, double* dC, double* dDskip,
                           double* dh0, double* dv0, int nthreads) {
  if (Bt < 0 || L < 0 || D < 0 || N < 0) return 1;
  if (Dskip && !dDskip) return 1;
  set_threads(nthreads);
  memset(dx, 0, sizeof(double) * (size_t)(Bt * L * D));
  memset(ddelta, 0, sizeof(double) * (size_t)(Bt * L * D));
  memset(dB, 0, sizeof(double) * (size_t)(Bt * L * N * 2));
  memset(dC, 0, sizeof(double) * (size_t)(Bt * L * N * 2));
  double* dA_rows = (double*)calloc((size_t)(Bt * D * N * 2) + 1, sizeof(double));
  double* dD_rows = (double*)calloc((size_t)(Bt * D) + 1, sizeof(double));
  if (!dA_rows || !dD_rows) { free(dA_rows); free(dD_rows); return 2; }
  int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < Bt; ++b) {
    double complex* hs = (double complex*)malloc(sizeof(double complex) * (size_t)(L + 1));
    if (!hs) {
#pragma omp atomic write
      failed = 1;
      continue;
    }
    for (int64_t d = 0; d < D; ++d) {
      for (int64_t n = 0; n < N; ++n) {
        const double complex An = cget(A, d * N + n);
        const int64_t s_i = (b * D + d) * N + n;
        double complex v = v0 ? cget(v0, s_i) : 0.0;
        double complex h = h0 ? cget(h0, s_i) : 0.0;
        hs[0] = h;
        for (int64_t t = 0; t < L; ++t) {
          double dt = delta[(b * L + t) * D + d];
          double xt = x[(b * L + t) * D + d];
          v = beta * v + alpha * dt * xt * cget(B, (b * L + t) * N + n);
          h = cexp(dt * An) * h + v;
          hs[t + 1] = h;
        }
        double complex gh_next = dlast_h ? cget(dlast_h, s_i) : 0.0, gv_next = 0.0;
        double complex a_next = 1.0;
        double complex dAn = 0.0;
        for (int64_t t = L - 1; t >= 0; --t) {
          int64_t i = (b * L + t) * D + d;
          int64_t j = (b * L + t) * N + n;
          double dt = delta[i], xt = x[i], dyt = dy[i];
          double complex a = cexp(dt * An);
          double complex Bj = cget(B, j), Cj = cget(C, j);
          double complex gh = dyt * conj(Cj) + conj(a_next) * gh_next;
          double complex gv = gh + beta * gv_next;
          if (t == L - 1 && dlast_v) gv += cget(dlast_v, s_i);
          double complex hprev = hs[t];
          double wr = creal(conj(gv) * Bj); /* Re(conj(gv) B) */
          dx[i] += alpha * dt * wr;
          ddelta[i] += alpha * xt * wr + creal(conj(gh) * An * a * hprev);
          dAn += conj(dt * a * hprev) * gh;
          double complex gB = alpha * dt * xt * gv;
          double complex gC = dyt * conj(hs[t + 1]);
          /* j belongs to batch row b: one thread writes it, channels in order */
          dB[2 * j] += creal(gB);
          dB[2 * j + 1] += cimag(gB);
          dC[2 * j] += creal(gC);
          dC[2 * j + 1] += cimag(gC);
          gh_next = gh;
          gv_next = gv;
          a_next = a;
        }
        dA_rows[2 * ((b * D + d) * N + n)] = creal(dAn);
        dA_rows[2 * ((b * D + d) * N + n) + 1] = cimag(dAn);
        if (dh0)
          cput(dh0, s_i, L > 0 ? conj(a_next) * gh_next : (dlast_h ? cget(dlast_h, s_i) : 0.0));
        if (dv0) cput(dv0, s_i, L > 0 ? beta * gv_next : (dlast_v ? cget(dlast_v, s_i) : 0.0));
      }
      if (Dskip) {
        for (int64_t t = 0; t < L; ++t) {
          int64_t i = (b * L + t) * D + d;
          dx[i] += Dskip[d] * dy[i];
          dD_rows[b * D + d] += dy[i] * x[i];
        }
      }
    }
    free(hs);
  }
  if (failed) { free(dA_rows); free(dD_rows); return 2; }
  for (int64_t k = 0; k < D * N * 2; ++k) {
    double s = 0.0;
    for (int64_t b = 0; b < Bt; ++b) s += dA_rows[b * D * N * 2 + k];
    dA[k] = s;
  }
  if (Dskip) {
    for (int64_t d = 0; d < D; ++d) {
      double s = 0.0;
      for (int64_t b = 0; b < Bt; ++b) s += dD_rows[b * D + d];
      dDskip[d] = s;
    }
  }
  free(dA_rows);
  free(dD_rows);
  return 0;
}
