/*
 * dig_oracle.c -- plain, slow, fp64 CPU oracle for the DiG gated-linear-attention
 * token mixer and the SREM step (scan-direction reorient + 3x3 depthwise conv).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no header, helper or table with the HIP library.
 *
 * Sources followed (the pages of the DiG description):
 *   [GLA]  DiG study-group slides (docswell), slide "GLA の導入", eqs. (5)-(10):
 *          S_t = G_t (.) S_{t-1} + K_t^T V_t,  O_t = Q_t S_t,  R_t = Swish(X W_r + b_r),
 *          Y_t = (R_t (.) Norm(O_t)) W_O.
 *   [LIN]  DiG paper write-up (volcengine), section 2 "Linear Attention Transformer":
 *          the feature map is the identity and the normalizer is dropped.
 *   [TAU]  DiG paper write-up (volcengine), section 3 "Preliminaries": tau is a
 *          temperature on the sigmoid gate.
 *   [SREM] DiG study-group slides, slide "SREM の導入", and the write-up's section 3
 *          "DiG Block": reshape the sequence to 2-D, 3x3 depthwise conv, transpose the
 *          token matrix and flip the flattened sequence to set the next scan direction.
 *
 * Readings where the pages are garbled or silent (the same readings the library
 * takes):
 *   - gate: log(alpha) = logsigmoid(z) / tau, i.e. alpha = sigmoid(z)^(1/tau); the
 *     value-side gate beta is 1 (gate matrix G_t = diag(alpha_t) applied to rows).
 *   - head-wise RMSNorm over each head's d_v outputs, epsilon eps, weight gamma[d_v]
 *     shared by the heads; Swish(x) = x * sigmoid(x).
 *   - S_0 = 0 for every (image, head); the recurrence runs over the sequence in the
 *     order it is stored (its current scan order).
 *   - scan directions, on an H x W grid with canonical id c(i,j) = i*W + j:
 *       ROW(p) = p, ROW_REV(p) = L-1-p, COL(p) = (p mod H)*W + p div H,
 *       COL_REV(p) = COL(L-1-p); "x in order d" means x[p] is the token c = pi_d(p).
 *   - the depthwise conv acts on the current-order sequence reshaped row-major to
 *     (H, W) for ROW/ROW_REV and to (W, H) for COL/COL_REV, zero padding 1, optional
 *     per-channel bias, no activation, no residual.
 *
 * Every function below is the plain definition: the token-by-token recurrence,
 * the direct convolution, the analytic chain rule.  No chunking, blocking or
 * reordering.
 *
 * Layouts: GLA tensors are [B, L, H, d] (token-major), SREM tensors are [B, L, D].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX4(b, t, h, e, L, H, d) ((((size_t)(b) * (L) + (t)) * (H) + (h)) * (d) + (e))

/* ---------------------------------------------------------------- gate [GLA eq.5][TAU] */

/* logsigmoid(z) = -log(1 + exp(-z)), written so that neither branch overflows. */
double oref_logsigmoid(double z)
{
    if (z >= 0.0) return -log1p(exp(-z));
    return z - log1p(exp(z));
}

double oref_sigmoid(double z)
{
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* log(alpha) = logsigmoid(z) / tau for n elements. */
void oref_gate_logalpha(size_t n, const double *z, double tau, double *loga)
{
    for (size_t i = 0; i < n; ++i) loga[i] = oref_logsigmoid(z[i]) / tau;
}

/* --------------------------------------------------------- recurrence [GLA eqs.6-8][LIN] */

/*
 * o_pre[b,t,h,:] = (q_scale * q_t) S_t with S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,
 * S_{-1} = 0, alpha_t = exp(loga_t).  loga may be 0 (alpha = 1) or -INFINITY (alpha = 0).
 */
static void recur_unit(int L, int H, int dk, int dv, int b, int h,
                       const double *q, const double *k, const double *v,
                       const double *loga, double q_scale, double *o_pre)
{
    double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
    for (int t = 0; t < L; ++t) {
        const double *qt = q + IDX4(b, t, h, 0, L, H, dk);
        const double *kt = k + IDX4(b, t, h, 0, L, H, dk);
        const double *vt = v + IDX4(b, t, h, 0, L, H, dv);
        const double *gt = loga + IDX4(b, t, h, 0, L, H, dk);
        for (int c = 0; c < dk; ++c) {
            double a = exp(gt[c]);
            for (int e = 0; e < dv; ++e)
                S[(size_t)c * dv + e] = a * S[(size_t)c * dv + e] + kt[c] * vt[e];
        }
        double *ot = o_pre + IDX4(b, t, h, 0, L, H, dv);
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += (q_scale * qt[c]) * S[(size_t)c * dv + e];
            ot[e] = acc;
        }
    }
    free(S);
}

void oref_gla_recurrence(int B, int L, int H, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *loga, double q_scale, double *o_pre)
{
    int units = B * H;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u)
        recur_unit(L, H, dk, dv, u / H, u % H, q, k, v, loga, q_scale, o_pre);
}

/* ------------------------------------------------------ output stage [GLA eqs.9-10] */

/*
 * y = (o * rstd) (.) gamma (.) swish(r),  rstd = (mean_{e<dv} o_e^2 + eps)^(-1/2),
 * per (b, t, h).  gamma == NULL means ones.  rstd_out (optional) is [B, L, H].
 */
void oref_output_stage(int B, int L, int H, int dv, const double *o_pre, const double *r,
                       const double *gamma, double eps, double *y, double *rstd_out)
{
    size_t rows = (size_t)B * L * H;
    for (size_t row = 0; row < rows; ++row) {
        const double *o = o_pre + row * dv;
        const double *rr = r + row * dv;
        double ss = 0.0;
        for (int e = 0; e < dv; ++e) ss += o[e] * o[e];
        double rstd = 1.0 / sqrt(ss / dv + eps);
        if (rstd_out) rstd_out[row] = rstd;
        for (int e = 0; e < dv; ++e) {
            double g = gamma ? gamma[e] : 1.0;
            double sw = rr[e] * oref_sigmoid(rr[e]);
            y[row * dv + e] = o[e] * rstd * g * sw;
        }
    }
}

/* Whole forward: gate, recurrence, output stage.  o_pre and rstd are optional. */
void oref_gla_fwd(int B, int L, int H, int dk, int dv,
                  const double *q, const double *k, const double *v, const double *z,
                  const double *r, const double *gamma, double tau, double q_scale,
                  double eps, double *y, double *o_pre_opt, double *rstd_opt)
{
    size_t nk = (size_t)B * L * H * dk, nv = (size_t)B * L * H * dv;
    double *loga = (double *)malloc(sizeof(double) * nk);
    double *o = o_pre_opt ? o_pre_opt : (double *)malloc(sizeof(double) * nv);
    oref_gate_logalpha(nk, z, tau, loga);
    oref_gla_recurrence(B, L, H, dk, dv, q, k, v, loga, q_scale, o);
    oref_output_stage(B, L, H, dv, o, r, gamma, eps, y, rstd_opt);
    if (!o_pre_opt) free(o);
    free(loga);
}

/* ------------------------------------------------------- backward (chain rule) */

/*
 * Gradients of L = <dy, y> through the forward above, taking log(alpha) as the gate
 * input (dloga) and also z (dz = dloga * sigmoid(-z) / tau) when z != NULL.
 * dgamma (optional, [dv]) is overwritten with the sum over b, t, h.
 *
 * Output stage, with s = swish(r), n = o * rstd:
 *   dgamma_e += dy_e n_e s_e
 *   dr_e      = dy_e n_e gamma_e * sigmoid(r_e) (1 + r_e (1 - sigmoid(r_e)))
 *   dn_e      = dy_e gamma_e s_e
 *   do_e      = rstd (dn_e - n_e * mean_j(dn_j n_j))
 * Recurrence, reverse time with dS = 0:
 *   dS += q_scale q_t^T do_t;  dq_t = q_scale S_t do_t;  dk_t = dS v_t;  dv_t = k_t dS;
 *   dloga_t[c] = alpha_t[c] sum_e dS[c,e] S_{t-1}[c,e];  dS = diag(alpha_t) dS.
 */
static void bwd_unit(int L, int H, int dk, int dv, int b, int h,
                     const double *q, const double *k, const double *v, const double *loga,
                     const double *r, const double *gamma, double q_scale, double eps,
                     const double *dy, double *dq, double *dk_, double *dv_, double *dloga,
                     double *dr, double *dgamma_unit)
{
    size_t sz = (size_t)dk * dv;
    double *states = (double *)malloc(sizeof(double) * sz * (size_t)L);
    double *o = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *dO = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *dS = (double *)calloc(sz, sizeof(double));
    double *n = (double *)malloc(sizeof(double) * dv);
    double *dn = (double *)malloc(sizeof(double) * dv);

    /* forward, keeping every state S_t */
    {
        double *S = (double *)calloc(sz, sizeof(double));
        for (int t = 0; t < L; ++t) {
            const double *kt = k + IDX4(b, t, h, 0, L, H, dk);
            const double *vt = v + IDX4(b, t, h, 0, L, H, dv);
            const double *qt = q + IDX4(b, t, h, 0, L, H, dk);
            const double *gt = loga + IDX4(b, t, h, 0, L, H, dk);
            for (int c = 0; c < dk; ++c) {
                double a = exp(gt[c]);
                for (int e = 0; e < dv; ++e) S[c * dv + e] = a * S[c * dv + e] + kt[c] * vt[e];
            }
            memcpy(states + (size_t)t * sz, S, sizeof(double) * sz);
            for (int e = 0; e < dv; ++e) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += (q_scale * qt[c]) * S[c * dv + e];
                o[(size_t)t * dv + e] = acc;
            }
        }
        free(S);
    }

    /* output-stage backward */
    for (int t = 0; t < L; ++t) {
        const double *ot = o + (size_t)t * dv;
        const double *rt = r + IDX4(b, t, h, 0, L, H, dv);
        const double *dyt = dy + IDX4(b, t, h, 0, L, H, dv);
        double *drt = dr + IDX4(b, t, h, 0, L, H, dv);
        double ss = 0.0;
        for (int e = 0; e < dv; ++e) ss += ot[e] * ot[e];
        double rstd = 1.0 / sqrt(ss / dv + eps);
        double m = 0.0;
        for (int e = 0; e < dv; ++e) {
            double g = gamma ? gamma[e] : 1.0;
            double sg = oref_sigmoid(rt[e]);
            double s = rt[e] * sg;
            n[e] = ot[e] * rstd;
            dgamma_unit[e] += dyt[e] * n[e] * s;
            drt[e] = dyt[e] * n[e] * g * sg * (1.0 + rt[e] * (1.0 - sg));
            dn[e] = dyt[e] * g * s;
            m += dn[e] * n[e];
        }
        m /= dv;
        for (int e = 0; e < dv; ++e) dO[(size_t)t * dv + e] = rstd * (dn[e] - n[e] * m);
    }

    /* reverse-time recurrence */
    for (int t = L - 1; t >= 0; --t) {
        const double *qt = q + IDX4(b, t, h, 0, L, H, dk);
        const double *kt = k + IDX4(b, t, h, 0, L, H, dk);
        const double *vt = v + IDX4(b, t, h, 0, L, H, dv);
        const double *gt = loga + IDX4(b, t, h, 0, L, H, dk);
        const double *dot = dO + (size_t)t * dv;
        const double *St = states + (size_t)t * sz;
        const double *Sp = t > 0 ? states + (size_t)(t - 1) * sz : NULL;
        for (int c = 0; c < dk; ++c)
            for (int e = 0; e < dv; ++e) dS[c * dv + e] += q_scale * qt[c] * dot[e];
        for (int c = 0; c < dk; ++c) {
            double aq = 0.0, ak = 0.0, ag = 0.0;
            for (int e = 0; e < dv; ++e) {
                aq += St[c * dv + e] * dot[e];
                ak += dS[c * dv + e] * vt[e];
                if (Sp) ag += dS[c * dv + e] * Sp[c * dv + e];
            }
            dq[IDX4(b, t, h, c, L, H, dk)] = q_scale * aq;
            dk_[IDX4(b, t, h, c, L, H, dk)] = ak;
            dloga[IDX4(b, t, h, c, L, H, dk)] = exp(gt[c]) * ag;
        }
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += kt[c] * dS[c * dv + e];
            dv_[IDX4(b, t, h, e, L, H, dv)] = acc;
        }
        for (int c = 0; c < dk; ++c) {
            double a = exp(gt[c]);
            for (int e = 0; e < dv; ++e) dS[c * dv + e] *= a;
        }
    }
    free(states); free(o); free(dO); free(dS); free(n); free(dn);
}

void oref_gla_bwd_logalpha(int B, int L, int H, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *loga, const double *r, const double *gamma,
                           double q_scale, double eps, const double *dy,
                           double *dq, double *dk_, double *dv_, double *dloga, double *dr,
                           double *dgamma)
{
    int units = B * H;
    double *dg_units = (double *)calloc((size_t)units * dv, sizeof(double));
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u)
        bwd_unit(L, H, dk, dv, u / H, u % H, q, k, v, loga, r, gamma, q_scale, eps, dy,
                 dq, dk_, dv_, dloga, dr, dg_units + (size_t)u * dv);
    if (dgamma) {
        for (int e = 0; e < dv; ++e) dgamma[e] = 0.0;
        for (int u = 0; u < units; ++u)
            for (int e = 0; e < dv; ++e) dgamma[e] += dg_units[(size_t)u * dv + e];
    }
    free(dg_units);
}

/* Backward with gate logits z: dz = dloga * sigmoid(-z) / tau. */
void oref_gla_bwd(int B, int L, int H, int dk, int dv,
                  const double *q, const double *k, const double *v, const double *z,
                  const double *r, const double *gamma, double tau, double q_scale,
                  double eps, const double *dy, double *dq, double *dk_, double *dv_,
                  double *dz, double *dr, double *dgamma)
{
    size_t nk = (size_t)B * L * H * dk;
    double *loga = (double *)malloc(sizeof(double) * nk);
    double *dloga = (double *)malloc(sizeof(double) * nk);
    oref_gate_logalpha(nk, z, tau, loga);
    oref_gla_bwd_logalpha(B, L, H, dk, dv, q, k, v, loga, r, gamma, q_scale, eps, dy,
                          dq, dk_, dv_, dloga, dr, dgamma);
    for (size_t i = 0; i < nk; ++i) dz[i] = dloga[i] * oref_sigmoid(-z[i]) / tau;
    free(loga);
    free(dloga);
}

/* ------------------------------------------- value-side gate beta [GLA eq.5][TAU] */

/*
 * The general gate of eq. (5): G_t = alpha_t^T beta_t, an outer product of a key-side gate
 * alpha_t (d_k) and a value-side gate beta_t (d_v), both sigmoid(.)^(1/tau) of their logits:
 *   S_t = G_t (.) S_{t-1} + k_t^T v_t,  o_t = (q_scale q_t) S_t,  S_{-1} = 0,
 * with G_t[c,e] = alpha_t[c] beta_t[e].  loga is [B,L,H,d_k], logb is [B,L,H,d_v].
 * beta = 1 (logb = 0) is the recurrence above.
 */
static void recur_unit_beta(int L, int H, int dk, int dv, int b, int h,
                            const double *q, const double *k, const double *v,
                            const double *loga, const double *logb, double q_scale,
                            double *o_unit, double *states_opt)
{
    /* o_unit: this unit's [L][dv] outputs; states_opt: its [L][dk][dv] states S_t */
    size_t sz = (size_t)dk * dv;
    double *S = (double *)calloc(sz, sizeof(double));
    for (int t = 0; t < L; ++t) {
        const double *qt = q + IDX4(b, t, h, 0, L, H, dk);
        const double *kt = k + IDX4(b, t, h, 0, L, H, dk);
        const double *vt = v + IDX4(b, t, h, 0, L, H, dv);
        const double *ga = loga + IDX4(b, t, h, 0, L, H, dk);
        const double *gb = logb + IDX4(b, t, h, 0, L, H, dv);
        for (int c = 0; c < dk; ++c)
            for (int e = 0; e < dv; ++e) {
                double g = exp(ga[c]) * exp(gb[e]);
                S[(size_t)c * dv + e] = g * S[(size_t)c * dv + e] + kt[c] * vt[e];
            }
        if (states_opt) memcpy(states_opt + (size_t)t * sz, S, sizeof(double) * sz);
        double *ot = o_unit + (size_t)t * dv;
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += (q_scale * qt[c]) * S[(size_t)c * dv + e];
            ot[e] = acc;
        }
    }
    free(S);
}

/* Whole forward with both gates: gate logits z (keys) and w (values), recurrence, output
 * stage.  o_pre and rstd are optional. */
void oref_gla_fwd_beta(int B, int L, int H, int dk, int dv,
                       const double *q, const double *k, const double *v, const double *z,
                       const double *w, const double *r, const double *gamma, double tau,
                       double q_scale, double eps, double *y, double *o_pre_opt,
                       double *rstd_opt)
{
    size_t nk = (size_t)B * L * H * dk, nv = (size_t)B * L * H * dv;
    double *loga = (double *)malloc(sizeof(double) * nk);
    double *logb = (double *)malloc(sizeof(double) * nv);
    double *o = o_pre_opt ? o_pre_opt : (double *)malloc(sizeof(double) * nv);
    oref_gate_logalpha(nk, z, tau, loga);
    oref_gate_logalpha(nv, w, tau, logb);
    int units = B * H;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u) {
        int b = u / H, h = u % H;
        double *ou = (double *)malloc(sizeof(double) * (size_t)L * dv);
        recur_unit_beta(L, H, dk, dv, b, h, q, k, v, loga, logb, q_scale, ou, NULL);
        for (int t = 0; t < L; ++t)
            memcpy(o + IDX4(b, t, h, 0, L, H, dv), ou + (size_t)t * dv, sizeof(double) * dv);
        free(ou);
    }
    oref_output_stage(B, L, H, dv, o, r, gamma, eps, y, rstd_opt);
    if (!o_pre_opt) free(o);
    free(loga);
    free(logb);
}

/*
 * Backward with both gates, L = <dy, y>.  The output stage is the one of bwd_unit; the
 * recurrence runs in reverse time with dS = 0:
 *   dS += q_scale q_t^T do_t;  dq_t = q_scale S_t do_t;  dk_t = dS v_t;  dv_t = k_t dS;
 *   dloga_t[c] = sum_e G_t[c,e] dS[c,e] S_{t-1}[c,e];
 *   dlogb_t[e] = sum_c G_t[c,e] dS[c,e] S_{t-1}[c,e];
 *   dS = G_t (.) dS.
 * dz = dloga sigmoid(-z) / tau and dw = dlogb sigmoid(-w) / tau.
 */
static void bwd_unit_beta(int L, int H, int dk, int dv, int b, int h,
                          const double *q, const double *k, const double *v,
                          const double *loga, const double *logb, const double *r,
                          const double *gamma, double q_scale, double eps, const double *dy,
                          double *dq, double *dk_, double *dv_, double *dloga, double *dlogb,
                          double *dr, double *dgamma_unit)
{
    size_t sz = (size_t)dk * dv;
    double *states = (double *)malloc(sizeof(double) * sz * (size_t)L);
    double *o = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *dO = (double *)malloc(sizeof(double) * (size_t)L * dv);
    double *dS = (double *)calloc(sz, sizeof(double));

    /* forward, keeping every state S_t (o is this unit's [L][dv] slice) */
    recur_unit_beta(L, H, dk, dv, b, h, q, k, v, loga, logb, q_scale, o, states);

    /* output-stage backward (as in bwd_unit) */
    for (int t = 0; t < L; ++t) {
        const double *ot = o + (size_t)t * dv;
        const double *rt = r + IDX4(b, t, h, 0, L, H, dv);
        const double *dyt = dy + IDX4(b, t, h, 0, L, H, dv);
        double *drt = dr + IDX4(b, t, h, 0, L, H, dv);
        double ss = 0.0;
        for (int e = 0; e < dv; ++e) ss += ot[e] * ot[e];
        double rstd = 1.0 / sqrt(ss / dv + eps);
        double m = 0.0;
        for (int e = 0; e < dv; ++e) {
            double g = gamma ? gamma[e] : 1.0;
            double sg = oref_sigmoid(rt[e]);
            double s = rt[e] * sg;
            double n = ot[e] * rstd;
            dgamma_unit[e] += dyt[e] * n * s;
            drt[e] = dyt[e] * n * g * sg * (1.0 + rt[e] * (1.0 - sg));
            m += dyt[e] * g * s * n;
        }
        m /= dv;
        for (int e = 0; e < dv; ++e) {
            double g = gamma ? gamma[e] : 1.0;
            double s = rt[e] * oref_sigmoid(rt[e]);
            dO[(size_t)t * dv + e] = rstd * (dyt[e] * g * s - ot[e] * rstd * m);
        }
    }

    /* reverse-time recurrence */
    for (int t = L - 1; t >= 0; --t) {
        const double *qt = q + IDX4(b, t, h, 0, L, H, dk);
        const double *kt = k + IDX4(b, t, h, 0, L, H, dk);
        const double *vt = v + IDX4(b, t, h, 0, L, H, dv);
        const double *ga = loga + IDX4(b, t, h, 0, L, H, dk);
        const double *gb = logb + IDX4(b, t, h, 0, L, H, dv);
        const double *dot = dO + (size_t)t * dv;
        const double *St = states + (size_t)t * sz;
        const double *Sp = t > 0 ? states + (size_t)(t - 1) * sz : NULL;
        for (int c = 0; c < dk; ++c)
            for (int e = 0; e < dv; ++e) dS[c * dv + e] += q_scale * qt[c] * dot[e];
        for (int c = 0; c < dk; ++c) {
            double aq = 0.0, ak = 0.0;
            for (int e = 0; e < dv; ++e) {
                aq += St[c * dv + e] * dot[e];
                ak += dS[c * dv + e] * vt[e];
            }
            dq[IDX4(b, t, h, c, L, H, dk)] = q_scale * aq;
            dk_[IDX4(b, t, h, c, L, H, dk)] = ak;
        }
        for (int e = 0; e < dv; ++e) {
            double acc = 0.0;
            for (int c = 0; c < dk; ++c) acc += kt[c] * dS[c * dv + e];
            dv_[IDX4(b, t, h, e, L, H, dv)] = acc;
        }
        for (int c = 0; c < dk; ++c) dloga[IDX4(b, t, h, c, L, H, dk)] = 0.0;
        for (int e = 0; e < dv; ++e) dlogb[IDX4(b, t, h, e, L, H, dv)] = 0.0;
        for (int c = 0; c < dk; ++c)
            for (int e = 0; e < dv; ++e) {
                double g = exp(ga[c]) * exp(gb[e]);
                double x = Sp ? g * dS[c * dv + e] * Sp[c * dv + e] : 0.0;
                dloga[IDX4(b, t, h, c, L, H, dk)] += x;
                dlogb[IDX4(b, t, h, e, L, H, dv)] += x;
                dS[c * dv + e] *= g;
            }
    }
    free(states); free(o); free(dO); free(dS);
}

void oref_gla_bwd_beta(int B, int L, int H, int dk, int dv,
                       const double *q, const double *k, const double *v, const double *z,
                       const double *w, const double *r, const double *gamma, double tau,
                       double q_scale, double eps, const double *dy, double *dq, double *dk_,
                       double *dv_, double *dz, double *dw, double *dr, double *dgamma)
{
    size_t nk = (size_t)B * L * H * dk, nv = (size_t)B * L * H * dv;
    int units = B * H;
    double *loga = (double *)malloc(sizeof(double) * nk);
    double *logb = (double *)malloc(sizeof(double) * nv);
    double *dloga = (double *)malloc(sizeof(double) * nk);
    double *dlogb = (double *)malloc(sizeof(double) * nv);
    double *dg_units = (double *)calloc((size_t)units * dv, sizeof(double));
    oref_gate_logalpha(nk, z, tau, loga);
    oref_gate_logalpha(nv, w, tau, logb);
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (int u = 0; u < units; ++u)
        bwd_unit_beta(L, H, dk, dv, u / H, u % H, q, k, v, loga, logb, r, gamma, q_scale, eps,
                      dy, dq, dk_, dv_, dloga, dlogb, dr, dg_units + (size_t)u * dv);
    if (dgamma) {
        for (int e = 0; e < dv; ++e) dgamma[e] = 0.0;
        for (int u = 0; u < units; ++u)
            for (int e = 0; e < dv; ++e) dgamma[e] += dg_units[(size_t)u * dv + e];
    }
    for (size_t i = 0; i < nk; ++i) dz[i] = dloga[i] * oref_sigmoid(-z[i]) / tau;
    for (size_t i = 0; i < nv; ++i) dw[i] = dlogb[i] * oref_sigmoid(-w[i]) / tau;
    free(loga); free(logb); free(dloga); free(dlogb); free(dg_units);
}

/* ------------------------------------------------------ scan directions [SREM] */

enum { OREF_ROW = 0, OREF_ROW_REV = 1, OREF_COL = 2, OREF_COL_REV = 3 };

/* pi_d(p): canonical id of the token at sequence position p in scan order d. */
int64_t oref_scan_canonical(int d, int64_t gh, int64_t gw, int64_t p)
{
    int64_t L = gh * gw;
    switch (d) {
    case OREF_ROW: return p;
    case OREF_ROW_REV: return L - 1 - p;
    case OREF_COL: return (p % gh) * gw + p / gh;
    case OREF_COL_REV: { int64_t s = L - 1 - p; return (s % gh) * gw + s / gh; }
    default: return -1;
    }
}

/* Fills perm[p] = pi_d(p) and inv[pi_d(p)] = p (either may be NULL). */
void oref_scan_perm(int d, int64_t gh, int64_t gw, int64_t *perm, int64_t *inv)
{
    int64_t L = gh * gw;
    for (int64_t p = 0; p < L; ++p) {
        int64_t c = oref_scan_canonical(d, gh, gw, p);
        if (perm) perm[p] = c;
        if (inv) inv[c] = p;
    }
}

/*
 * Reorient: y[b, p, :] = x[b, p_from(pi_to(p)), :] where p_from is the inverse of pi_from.
 * Byte copy of whole token rows (row_bytes = channels * element size): exact.
 */
void oref_reorient(int B, int64_t gh, int64_t gw, int64_t row_bytes, int from, int to,
                   const void *x, void *y)
{
    int64_t L = gh * gw;
    int64_t *inv_from = (int64_t *)malloc(sizeof(int64_t) * L);
    oref_scan_perm(from, gh, gw, NULL, inv_from);
    for (int b = 0; b < B; ++b)
        for (int64_t p = 0; p < L; ++p) {
            int64_t src = inv_from[oref_scan_canonical(to, gh, gw, p)];
            memcpy((char *)y + ((size_t)b * L + p) * row_bytes,
                   (const char *)x + ((size_t)b * L + src) * row_bytes, (size_t)row_bytes);
        }
    free(inv_from);
}

/* ---------------------------------------------------------- 3x3 depthwise conv [SREM] */

/* Grid shape the conv sees for a sequence stored in order d: (rows, cols). */
static void cur_grid(int d, int64_t gh, int64_t gw, int64_t *rows, int64_t *cols)
{
    if (d == OREF_COL || d == OREF_COL_REV) { *rows = gw; *cols = gh; }
    else { *rows = gh; *cols = gw; }
}

/*
 * y_conv[b, i*cols + j, c] = bias[c] + sum_{a,s in {-1,0,1}} w[c, a+1, s+1] x[b, (i+a)*cols + (j+s), c]
 * on the current-order grid (zero outside), then written in order `to`:
 * y[b, p, c] = y_conv[b, p_from(pi_to(p)), c].  w is [D, 3, 3]; bias may be NULL.
 */
void oref_dwconv3x3(int B, int64_t gh, int64_t gw, int D, int layout, int out_layout,
                    const double *x, const double *w, const double *bias, double *y)
{
    int64_t L = gh * gw, rows, cols;
    cur_grid(layout, gh, gw, &rows, &cols);
    double *yc = (double *)malloc(sizeof(double) * (size_t)L * D);
    int64_t *inv_from = (int64_t *)malloc(sizeof(int64_t) * L);
    oref_scan_perm(layout, gh, gw, NULL, inv_from);
    for (int b = 0; b < B; ++b) {
        const double *xb = x + (size_t)b * L * D;
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < cols; ++j)
                for (int c = 0; c < D; ++c) {
                    double acc = bias ? bias[c] : 0.0;
                    for (int a = -1; a <= 1; ++a)
                        for (int s = -1; s <= 1; ++s) {
                            int64_t ii = i + a, jj = j + s;
                            if (ii < 0 || ii >= rows || jj < 0 || jj >= cols) continue;
                            acc += w[(size_t)c * 9 + (a + 1) * 3 + (s + 1)] *
                                   xb[(size_t)(ii * cols + jj) * D + c];
                        }
                    yc[(size_t)(i * cols + j) * D + c] = acc;
                }
        for (int64_t p = 0; p < L; ++p) {
            int64_t src = inv_from[oref_scan_canonical(out_layout, gh, gw, p)];
            memcpy(y + ((size_t)b * L + p) * D, yc + (size_t)src * D, sizeof(double) * D);
        }
    }
    free(yc);
    free(inv_from);
}

/*
 * Backward of oref_dwconv3x3 for L = <dy, y>:
 *   dy_conv[p] = dy[p_to(pi_from(p))]   (undo the reorient)
 *   dx[i,j,c]  = sum_{a,s} w[c,a+1,s+1] dy_conv[i-a, j-s, c]
 *   dw[c,a+1,s+1] = sum_{b,i,j} dy_conv[i,j,c] x[i+a, j+s, c];  dbias[c] = sum dy.
 * dw and dbias (optional) are overwritten.
 */
void oref_dwconv3x3_bwd(int B, int64_t gh, int64_t gw, int D, int layout, int out_layout,
                        const double *x, const double *w, const double *dy,
                        double *dx, double *dw, double *dbias)
{
    int64_t L = gh * gw, rows, cols;
    cur_grid(layout, gh, gw, &rows, &cols);
    double *dyc = (double *)malloc(sizeof(double) * (size_t)L * D);
    int64_t *inv_to = (int64_t *)malloc(sizeof(int64_t) * L);
    oref_scan_perm(out_layout, gh, gw, NULL, inv_to);
    for (int c = 0; c < 9 * D; ++c) dw[c] = 0.0;
    if (dbias) for (int c = 0; c < D; ++c) dbias[c] = 0.0;
    for (int b = 0; b < B; ++b) {
        const double *xb = x + (size_t)b * L * D;
        for (int64_t p = 0; p < L; ++p) {
            int64_t src = inv_to[oref_scan_canonical(layout, gh, gw, p)];
            memcpy(dyc + (size_t)p * D, dy + ((size_t)b * L + src) * D, sizeof(double) * D);
        }
        for (int64_t i = 0; i < rows; ++i)
            for (int64_t j = 0; j < cols; ++j)
                for (int c = 0; c < D; ++c) {
                    double acc = 0.0, g = dyc[(size_t)(i * cols + j) * D + c];
                    if (dbias) dbias[c] += g;
                    for (int a = -1; a <= 1; ++a)
                        for (int s = -1; s <= 1; ++s) {
                            int64_t ii = i - a, jj = j - s;
                            if (ii >= 0 && ii < rows && jj >= 0 && jj < cols)
                                acc += w[(size_t)c * 9 + (a + 1) * 3 + (s + 1)] *
                                       dyc[(size_t)(ii * cols + jj) * D + c];
                            int64_t xi = i + a, xj = j + s;
                            if (xi >= 0 && xi < rows && xj >= 0 && xj < cols)
                                dw[(size_t)c * 9 + (a + 1) * 3 + (s + 1)] +=
                                    g * xb[(size_t)(xi * cols + xj) * D + c];
                        }
                    dx[((size_t)b * L + i * cols + j) * D + c] = acc;
                }
    }
    free(dyc);
    free(inv_to);
}

/*
 * Linear projection around the token mixer (DiG study-group slides, slide introducing GLA,
 * eqs. (5), (9), (10): Q = X W_Q, K = X W_K, V = X W_V, the gate logits, R = X W_r + b_r and
 * Y = (...) W_O), with the weight stored as (out features x in features):
 *   c[i][j] = sum_l a[i][l] w[j][l] + bias[j]          (bias may be NULL: no bias)
 * a [m][k], w [n][k], c [m][n], fp64, the plain definition (rows in parallel).
 */
void oref_linear(int64_t m, int64_t k, int64_t n, const double *a, const double *w,
                 const double *bias, double *c)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t l = 0; l < k; ++l)
                acc += a[(size_t)i * k + l] * w[(size_t)j * k + l];
            c[(size_t)i * n + j] = acc + (bias ? bias[j] : 0.0);
        }
}

/*
 * The adaptive normalisation of a DiG block (slides Figure 4: RMS Norm, then Scale & Shift by
 * the gamma, beta regressed from the conditioning; write-up section 3 "DiG Block"), per row i
 * of D values, image g = i / rows_per_group:
 *   h[i][j] = x[i][j] / sqrt(mean_l x[i][l]^2 + eps) * scale[g][j] + shift[g][j]
 * scale and shift rows are mod_ld apart.  fp64, the plain definition.
 */
void oref_rmsnorm_modulate(int64_t rows, int64_t D, int64_t rows_per_group, const double *x,
                           const double *scale, const double *shift, int64_t mod_ld,
                           double eps, double *h)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const double *xr = x + (size_t)i * D;
        double ss = 0.0;
        for (int64_t j = 0; j < D; ++j) ss += xr[j] * xr[j];
        const double inv = 1.0 / sqrt(ss / (double)D + eps);
        const int64_t g = i / rows_per_group;
        for (int64_t j = 0; j < D; ++j)
            h[(size_t)i * D + j] = xr[j] * inv * scale[(size_t)g * mod_ld + j] +
                                   shift[(size_t)g * mod_ld + j];
    }
}

/* GELU of the DiG feedforward, exact form: y = x Phi(x) = x (1 + erf(x / sqrt(2))) / 2. */
void oref_gelu(int64_t n, const double *x, double *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = 0.5 * x[i] * (1.0 + erf(x[i] / sqrt(2.0)));
}

/* SiLU applied to the conditioning before the adaLN regression: y = x / (1 + e^{-x}). */
void oref_silu(int64_t n, const double *x, double *y)
{
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] / (1.0 + exp(-x[i]));
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
