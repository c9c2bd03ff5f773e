/*
 * Plain fp64 CPU oracle for causal kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; it is written directly from the pages' equations.
 *
 * Sources (page titles, sections, equations):
 *   [LA]  "2.2 Linear Attention" (efficient2 page): feature-mapped Q' = phi(Q),
 *         K' = phi(K) (text before eq 6); eq 6 (D^-1 (Q'(K'^T V)));
 *         eqs 7-8 (running sums mu_j, nu_j); eq 9 and its causal form
 *         (readout q'_j mu_j / q'_j nu_j); eqs 10-11 (decayed sums with a).
 *   [KM]  "3.2 Reducing d" (efficient1 page): eqs 22-27, the kernelized
 *         attention c_i = phi(q_i) (sum phi(k_j)^T v_j) / phi(q_i) (sum phi(k_j)^T),
 *         and the remark that both sums are kept and updated as new keys and
 *         values arrive.
 *   [RF]  "Linear attention research 2026" page, section on Performer random
 *         features: phi(x) = exp(x . omega - |x|^2 / 2) / sqrt(m); section on
 *         the Linear Transformer: phi(x) = elu(x) + 1.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes): elu's alpha is 1; the mask is inclusive (position i sees itself);
 * the prefill state starts at zero; no epsilon is added to the denominator;
 * the decode readout is taken after the state update; omega [d, m] is an
 * input shared by every batch and head; decay is one value a per head.
 *
 * Arithmetic is IEEE fp64 throughout, in the order the equations state: the
 * literal per-position recurrence, no chunking, no blocking, no reordering.
 * Inputs arrive already widened to fp64 from whatever storage precision the
 * caller used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_MAP_IDENTITY = 0, ORC_MAP_ELU1 = 1, ORC_MAP_PERFORMER = 2 };

/* [RF] Linear Transformer: phi(x) = elu(x) + 1 with alpha = 1, i.e. x + 1 for
 * x > 0 and exp(x) otherwise. */
static double elu_plus_one(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* Feature map of one row x[0..d) into y[0..dfeat).  d is the width of the
 * q/k rows as stored.
 *   IDENTITY : y = x (dfeat == d), the caller already feature-mapped.
 *   ELU1     : y_c = elu(x_c) + 1 (dfeat == d)                       [RF]
 *   PERFORMER: u_r = sum_c x_c omega[c][r]; y_r = exp(u_r - |x|^2/2)/sqrt(m)
 *              with omega stored row-major [d][m] (dfeat == m)       [RF]   */
static void feature_row(const double *x, double *y, int d, int dfeat, int map,
                        const double *omega) {
  if (map == ORC_MAP_IDENTITY) {
    for (int c = 0; c < d; ++c) y[c] = x[c];
  } else if (map == ORC_MAP_ELU1) {
    for (int c = 0; c < d; ++c) y[c] = elu_plus_one(x[c]);
  } else {
    double sq = 0.0;
    for (int c = 0; c < d; ++c) sq += x[c] * x[c];
    const double inv_sqrt_m = 1.0 / sqrt((double)dfeat);
    for (int r = 0; r < dfeat; ++r) {
      double u = 0.0;
      for (int c = 0; c < d; ++c) u += x[c] * omega[(int64_t)c * dfeat + r];
      y[r] = exp(u - 0.5 * sq) * inv_sqrt_m;
    }
  }
}

/* Row-wise feature map over `rows` rows: x [rows][d] -> y [rows][dfeat]. */
void oracle_featmap(const double *x, double *y, const double *omega,
                    int64_t rows, int d, int dfeat, int map) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < rows; ++i)
    feature_row(x + i * d, y + i * dfeat, d, dfeat, map, omega);
}

/* One state update, eqs 7-8 (no decay) or eqs 10-11 (decay a):
 *   mu <- a mu + (1-a) k'^T v,   nu <- a nu + (1-a) k'
 * mu is [dfeat][d] row-major: mu[f][e] accumulates k'_f v_e.            [LA] */
static void state_update(double *mu, double *nu, const double *kf,
                         const double *v, int d, int dfeat, int has_decay,
                         double a) {
  if (has_decay) {
    const double b = 1.0 - a;
    for (int f = 0; f < dfeat; ++f) {
      for (int e = 0; e < d; ++e)
        mu[f * d + e] = a * mu[f * d + e] + b * kf[f] * v[e];
      nu[f] = a * nu[f] + b * kf[f];
    }
  } else {
    for (int f = 0; f < dfeat; ++f) {
      for (int e = 0; e < d; ++e) mu[f * d + e] += kf[f] * v[e];
      nu[f] += kf[f];
    }
  }
}

/* Readout, eq 9 (and its causal form): out = (q' mu) / (q' . nu).  No epsilon:
 * IEEE division, so a zero denominator gives inf or nan.                 [LA] */
static void readout(const double *mu, const double *nu, const double *qf,
                    double *out, int d, int dfeat) {
  double den = 0.0;
  for (int f = 0; f < dfeat; ++f) den += qf[f] * nu[f];
  for (int e = 0; e < d; ++e) {
    double num = 0.0;
    for (int f = 0; f < dfeat; ++f) num += qf[f] * mu[f * d + e];
    out[e] = num / den;
  }
}

/* Full forward pass over B*H independent (batch, head) units.
 *   q, k : [B][H][n][dqk]    v, out : [B][H][n][d]
 *   dqk = d for ELU1 and PERFORMER, dqk = dfeat for IDENTITY.
 *   omega: [d][dfeat] (PERFORMER only), decay: [H] or NULL (eqs 7-8).
 * causal = 1: out_j reads mu_j, nu_j after position j is added (inclusive).
 * causal = 0: every out_j reads the final mu_n, nu_n (eq 9).
 * The state starts at zero for every unit.                                 */
void oracle_forward(const double *q, const double *k, const double *v,
                    double *out, int B, int H, int64_t n, int d, int dqk,
                    int dfeat, int map, const double *omega,
                    const double *decay, int causal) {
  const int64_t units = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    const double *qu = q + u * n * dqk, *ku = k + u * n * dqk;
    const double *vu = v + u * n * d;
    double *ou = out + u * n * d;
    double *mu = (double *)calloc((size_t)dfeat * d, sizeof(double));
    double *nu = (double *)calloc((size_t)dfeat, sizeof(double));
    double *qf = (double *)malloc(sizeof(double) * dfeat);
    double *kf = (double *)malloc(sizeof(double) * dfeat);
    const int has_decay = decay != NULL;
    const double a = has_decay ? decay[h] : 1.0;
    for (int64_t j = 0; j < n; ++j) {
      feature_row(ku + j * dqk, kf, dqk, dfeat, map, omega);
      state_update(mu, nu, kf, vu + j * d, d, dfeat, has_decay, a);
      if (causal) {
        feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
        readout(mu, nu, qf, ou + j * d, d, dfeat);
      }
    }
    if (!causal) {
      for (int64_t j = 0; j < n; ++j) {
        feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
        readout(mu, nu, qf, ou + j * d, d, dfeat);
      }
    }
    free(mu); free(nu); free(qf); free(kf);
  }
}

/* One decode step per (sequence, head) unit: mu, nu hold the running sums of
 * everything seen so far; a new (q, k, v) arrives; the sums are updated in
 * place (eqs 7-8 or 10-11) and the new token's output is read out from the
 * updated sums ([KM] remark after eq 27; [LA] causal form of eq 9).
 *   mu: [S][H][dfeat][d]  nu: [S][H][dfeat]  q, k: [S][H][dqk]
 *   v, out: [S][H][d]   (dqk = dfeat for IDENTITY, d otherwise)            */
void oracle_decode(double *mu, double *nu, const double *q, const double *k,
                   const double *v, double *out, int S, int H, int d, int dqk,
                   int dfeat, int map, const double *omega,
                   const double *decay) {
  const int64_t units = (int64_t)S * H;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    double *qf = (double *)malloc(sizeof(double) * dfeat);
    double *kf = (double *)malloc(sizeof(double) * dfeat);
    const int has_decay = decay != NULL;
    const double a = has_decay ? decay[h] : 1.0;
    double *muu = mu + u * (int64_t)dfeat * d, *nuu = nu + u * (int64_t)dfeat;
    feature_row(k + u * dqk, kf, dqk, dfeat, map, omega);
    state_update(muu, nuu, kf, v + u * d, d, dfeat, has_decay, a);
    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);
    readout(muu, nuu, qf, out + u * d, d, dfeat);
    free(qf); free(kf);
  }
}

/* ------------------------------------------------------------------------
 * Diagonal and input-dependent decay.
 *
 * [SSM]  "2.3 State-Space Models" (efficient2 page): the discretised state
 *        update z_t = z_{t-1} A + s_t B (eq 14), unrolled with powers of A
 *        (eqs 16-17), and A diagonalised to Lambda (eqs 21-25), so every
 *        state channel decays by its own factor.
 * [MB]   "Linear attention research 2026" page, Mamba's selective
 *        mechanism: the decay is input-dependent, dA = exp(A delta_t).
 *
 * Reading (listed in the design notes): the log decay lam = log(gamma) is
 * given per state row f (feature channel) and/or per position j; the
 * update is eqs 10-11 with a replaced by gamma_{j,f} = exp(lam_{j,f}) on
 * row f, and the input weight is 1 - gamma_{j,f}, the (1 - a) of eqs
 * 10-11 (the zero-order-hold input weight of eq 14 up to a constant that
 * cancels in the ratio):
 *   mu_j[f][e] = gamma mu_{j-1}[f][e] + (1 - gamma) k'_{j,f} v_{j,e}
 *   nu_j[f]    = gamma nu_{j-1}[f]    + (1 - gamma) k'_{j,f}
 * The readout is eq 9 (causal form), unchanged.
 * Layouts of lam (fp64 here), by mode:
 *   ORC_LD_CHANNEL  : [H][dfeat], the same at every position (eqs 21-25)
 *   ORC_LD_POSITION : [B][H][n] (decode: [S][H]), the same for every row
 *   ORC_LD_BOTH     : [B][H][n][dfeat] (decode: [S][H][dfeat])
 * ------------------------------------------------------------------------ */
enum { ORC_LD_CHANNEL = 0, ORC_LD_POSITION = 1, ORC_LD_BOTH = 2 };

/* log decay of row f at position j of unit u (head h) */
static double lam_at(const double *lam, int mode, int64_t u, int h,
                     int64_t j, int64_t n, int f, int dfeat) {
  if (mode == ORC_LD_CHANNEL) return lam[(int64_t)h * dfeat + f];
  if (mode == ORC_LD_POSITION) return lam[u * n + j];
  return lam[(u * n + j) * dfeat + f];
}

/* One gated update of every state row (the recurrence above). */
static void gated_update(double *mu, double *nu, const double *kf,
                         const double *v, int d, int dfeat, const double *lam,
                         int mode, int64_t u, int h, int64_t j, int64_t n) {
  for (int f = 0; f < dfeat; ++f) {
    const double g = exp(lam_at(lam, mode, u, h, j, n, f, dfeat));
    const double b = 1.0 - g;
    for (int e = 0; e < d; ++e)
      mu[f * d + e] = g * mu[f * d + e] + b * kf[f] * v[e];
    nu[f] = g * nu[f] + b * kf[f];
  }
}

/* Forward with the gated recurrence, over B*H units from a zero state;
 * arguments as oracle_forward, with lam and its mode in place of decay. */
void oracle_forward_gated(const double *q, const double *k, const double *v,
                          double *out, int B, int H, int64_t n, int d,
                          int dqk, int dfeat, int map, const double *omega,
                          const double *lam, int mode, int causal) {
  const int64_t units = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    const double *qu = q + u * n * dqk, *ku = k + u * n * dqk;
    const double *vu = v + u * n * d;
    double *ou = out + u * n * d;
    double *mu = (double *)calloc((size_t)dfeat * d, sizeof(double));
    double *nu = (double *)calloc((size_t)dfeat, sizeof(double));
    double *qf = (double *)malloc(sizeof(double) * dfeat);
    double *kf = (double *)malloc(sizeof(double) * dfeat);
    for (int64_t j = 0; j < n; ++j) {
      feature_row(ku + j * dqk, kf, dqk, dfeat, map, omega);
      gated_update(mu, nu, kf, vu + j * d, d, dfeat, lam, mode, u, h, j, n);
      if (causal) {
        feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
        readout(mu, nu, qf, ou + j * d, d, dfeat);
      }
    }
    /* non-causal: every row reads the final sums (eq 9) */
    for (int64_t j = 0; !causal && j < n; ++j) {
      feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
      readout(mu, nu, qf, ou + j * d, d, dfeat);
    }
    free(mu); free(nu); free(qf); free(kf);
  }
}

/* One decode step with the gated update; lam is [H][dfeat] (CHANNEL),
 * [S][H] (POSITION: one value per unit) or [S][H][dfeat] (BOTH). */
void oracle_decode_gated(double *mu, double *nu, const double *q,
                         const double *k, const double *v, double *out, int S,
                         int H, int d, int dqk, int dfeat, int map,
                         const double *omega, const double *lam, int mode) {
  const int64_t units = (int64_t)S * H;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    double *qf = (double *)malloc(sizeof(double) * dfeat);
    double *kf = (double *)malloc(sizeof(double) * dfeat);
    double *muu = mu + u * (int64_t)dfeat * d, *nuu = nu + u * (int64_t)dfeat;
    feature_row(k + u * dqk, kf, dqk, dfeat, map, omega);
    /* a decode step is position 0 of a one-position sequence */
    gated_update(muu, nuu, kf, v + u * d, d, dfeat, lam, mode, u, h, 0, 1);
    feature_row(q + u * dqk, qf, dqk, dfeat, map, omega);
    readout(muu, nuu, qf, out + u * d, d, dfeat);
    free(qf); free(kf);
  }
}

/* ------------------------------------------------------------------------
 * Gradients (backward pass) of the causal forward.
 *
 * The pages give the forward only; training through it ("Linear attention
 * research 2026" page, its closing section on parallel training of the
 * recurrent forms) needs the derivatives of out with respect to q, k, v.
 * They are written here as the adjoint of the literal recurrence above,
 * step by step (reverse-mode differentiation through the positions), in
 * two sweeps so that no state has to be stored per position:
 *
 *   forward sweep, j = 1 .. n (the recurrence of eqs 7-8 / 10-11):
 *     num_j = q'_j mu_j,  den_j = q'_j . nu_j,  out_j = num_j / den_j
 *     dnum_j = dout_j / den_j,  dden_j = -(dout_j . num_j) / den_j^2
 *     dq'_j  = mu_j dnum_j + nu_j dden_j        (mu_j row f: sum over e)
 *   backward sweep, j = n .. 1, adjoint states M (d' x d) and Z (d'):
 *     M += q'_j dnum_j^T,  Z += q'_j dden_j     (the readout at j)
 *     dk'_j = b (M v_j + Z),  dv_j = b M^T k'_j (the update at j)
 *     M <- g M,  Z <- g Z                       (mu_j = g mu_{j-1} + ...)
 *   with g = b = 1 (eqs 7-8) or g = a, b = 1 - a (eqs 10-11); then the
 *   chain rule through the feature map, per element:
 *     ELU1: dx = dx' (x > 0) or dx' e^x (x <= 0);  IDENTITY: dx = dx';
 *     PERFORMER: dx_c = sum_r dx'_r phi_r (omega[c][r] - x_c).
 * Layouts as oracle_forward; dout, dq, dk, dv have the shapes of out, q,
 * k, v.  Causal only.
 * ------------------------------------------------------------------------ */

/* d phi(x) / d x applied to the feature gradient gf (d' values) of the row
 * x (d values): gx[c] = sum_r gf[r] d phi_r / d x_c. */
static void feature_row_grad(const double *x, const double *gf, double *gx,
                             int d, int dfeat, int map, const double *omega) {
  if (map == ORC_MAP_IDENTITY) {
    for (int c = 0; c < d; ++c) gx[c] = gf[c];
  } else if (map == ORC_MAP_ELU1) {
    for (int c = 0; c < d; ++c) gx[c] = x[c] > 0.0 ? gf[c] : gf[c] * exp(x[c]);
  } else {
    double *phi = (double *)malloc(sizeof(double) * dfeat);
    feature_row(x, phi, d, dfeat, map, omega);
    double s = 0.0;   /* sum_r gf_r phi_r */
    for (int r = 0; r < dfeat; ++r) s += gf[r] * phi[r];
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int r = 0; r < dfeat; ++r)
        acc += gf[r] * phi[r] * omega[c * (int64_t)dfeat + r];
      gx[c] = acc - x[c] * s;
    }
    free(phi);
  }
}

/* The adjoint for one unit.  Decay: per head (has_decay, a; none: a = 1,
 * input weight 1) or, with lam, the gated decay g = exp(lam) and input
 * weight 1 - g of each position and state row (lam and mode as
 * oracle_forward_gated).  Going backward, the adjoint states take row f of
 * position j's input weight for dk, dv at j, then decay by row f of
 * position j's decay on their way to j - 1 (d mu_j / d mu_{j-1} = g_j).
 * The decay itself is not differentiated. */
static void backward_unit(const double *qu, const double *ku, const double *vu,
                          const double *gu, double *dqu, double *dku,
                          double *dvu, int64_t n, int d, int dqk, int dfeat,
                          int map, const double *omega, int has_decay,
                          double a, const double *lam, int mode, int64_t u,
                          int h) {
  double *mu = (double *)calloc((size_t)dfeat * d, sizeof(double));
  double *nu = (double *)calloc((size_t)dfeat, sizeof(double));
  double *qf = (double *)malloc(sizeof(double) * dfeat);
  double *kf = (double *)malloc(sizeof(double) * dfeat);
  double *gf = (double *)malloc(sizeof(double) * dfeat);
  double *gw = (double *)malloc(sizeof(double) * dfeat);  /* decay of row f */
  double *bw = (double *)malloc(sizeof(double) * dfeat);  /* input weight */
  /* per position: dnum (d) and dden (1), kept for the backward sweep */
  double *dnum = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *dden = (double *)malloc(sizeof(double) * (size_t)n);
  /* forward sweep */
  for (int64_t j = 0; j < n; ++j) {
    feature_row(ku + j * dqk, kf, dqk, dfeat, map, omega);
    if (lam)
      gated_update(mu, nu, kf, vu + j * d, d, dfeat, lam, mode, u, h, j, n);
    else
      state_update(mu, nu, kf, vu + j * d, d, dfeat, has_decay, a);
    feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
    double den = 0.0;
    for (int f = 0; f < dfeat; ++f) den += qf[f] * nu[f];
    double dn = 0.0;   /* dout_j . num_j */
    for (int e = 0; e < d; ++e) {
      double num = 0.0;
      for (int f = 0; f < dfeat; ++f) num += mu[f * d + e] * qf[f];
      dnum[j * d + e] = gu[j * d + e] / den;
      dn += gu[j * d + e] * num;
    }
    dden[j] = -dn / (den * den);
    for (int f = 0; f < dfeat; ++f) {
      double acc = nu[f] * dden[j];
      for (int e = 0; e < d; ++e) acc += mu[f * d + e] * dnum[j * d + e];
      gf[f] = acc;
    }
    feature_row_grad(qu + j * dqk, gf, dqu + j * dqk, dqk, dfeat, map, omega);
  }
  /* backward sweep: adjoint states M (reusing mu) and Z (reusing nu) */
  memset(mu, 0, sizeof(double) * (size_t)dfeat * d);
  memset(nu, 0, sizeof(double) * (size_t)dfeat);
  for (int64_t j = n - 1; j >= 0; --j) {
    for (int f = 0; f < dfeat; ++f) {
      gw[f] = lam ? exp(lam_at(lam, mode, u, h, j, n, f, dfeat))
                  : has_decay ? a : 1.0;
      bw[f] = lam || has_decay ? 1.0 - gw[f] : 1.0;
    }
    feature_row(qu + j * dqk, qf, dqk, dfeat, map, omega);
    for (int f = 0; f < dfeat; ++f) {
      for (int e = 0; e < d; ++e) mu[f * d + e] += qf[f] * dnum[j * d + e];
      nu[f] += qf[f] * dden[j];
    }
    feature_row(ku + j * dqk, kf, dqk, dfeat, map, omega);
    for (int f = 0; f < dfeat; ++f) {
      const double b = bw[f];
      double acc = nu[f];
      for (int e = 0; e < d; ++e) acc += mu[f * d + e] * vu[j * d + e];
      gf[f] = b * acc;
    }
    feature_row_grad(ku + j * dqk, gf, dku + j * dqk, dqk, dfeat, map, omega);
    for (int e = 0; e < d; ++e) {
      double acc = 0.0;
      for (int f = 0; f < dfeat; ++f) acc += mu[f * d + e] * kf[f] * bw[f];
      dvu[j * d + e] = acc;
    }
    for (int f = 0; f < dfeat; ++f) {
      for (int e = 0; e < d; ++e) mu[f * d + e] *= gw[f];
      nu[f] *= gw[f];
    }
  }
  free(mu); free(nu); free(qf); free(kf); free(gf); free(gw); free(bw);
  free(dnum); free(dden);
}

void oracle_backward(const double *q, const double *k, const double *v,
                     const double *dout, double *dq, double *dk, double *dv,
                     int B, int H, int64_t n, int d, int dqk, int dfeat,
                     int map, const double *omega, const double *decay) {
  const int64_t units = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    backward_unit(q + u * n * dqk, k + u * n * dqk, v + u * n * d,
                  dout + u * n * d, dq + u * n * dqk, dk + u * n * dqk,
                  dv + u * n * d, n, d, dqk, dfeat, map, omega, decay != NULL,
                  decay ? decay[h] : 1.0, NULL, 0, u, h);
  }
}

/* Gradients of the causal forward with the gated recurrence (lam and mode
 * as oracle_forward_gated): the adjoint above with each position's and
 * state row's decay in place of one per head. */
void oracle_backward_gated(const double *q, const double *k, const double *v,
                           const double *dout, double *dq, double *dk,
                           double *dv, int B, int H, int64_t n, int d,
                           int dqk, int dfeat, int map, const double *omega,
                           const double *lam, int mode) {
  const int64_t units = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    const int h = (int)(u % H);
    backward_unit(q + u * n * dqk, k + u * n * dqk, v + u * n * d,
                  dout + u * n * d, dq + u * n * dqk, dk + u * n * dqk,
                  dv + u * n * d, n, d, dqk, dfeat, map, omega, 0, 1.0, lam,
                  mode, u, h);
  }
}

/* Number of OpenMP threads a parallel region here would use (1 without
 * OpenMP); reported beside the oracle's timing. */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
int oracle_num_threads(void) { return 1; }
#endif
