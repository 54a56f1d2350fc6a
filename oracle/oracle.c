/*
 * oracle.c -- fp64 CPU reference implementation (TEST INFRASTRUCTURE ONLY).
 *
 * Written from the pages' definitions, one routine per definition, with no
 * blocking, chunking or reordering beyond what each definition states.
 * See oracle.h for the sources, the array conventions and the feature order.
 * Shares no code with the HIP library.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_features(int d) { return 1 + d + d * d; }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [BASED s4 "Taylor Linear Attention"]: 2nd-order Taylor feature map on the
 * projected dim d.  The input is pre-scaled by d^(-1/4) so that
 * phi(q).phi(k) = 1 + (q.k)/sqrt(d) + ((q.k)/sqrt(d))^2 / 2. */
void oracle_taylor_features(const double *x, int d, double *out) {
    const double pre = pow((double)d, -0.25);
    const double inv_sqrt2 = 1.0 / sqrt(2.0);
    out[0] = 1.0;
    for (int a = 0; a < d; ++a) out[1 + a] = x[a] * pre;
    for (int a = 0; a < d; ++a)
        for (int b = 0; b < d; ++b)
            out[1 + d + a * d + b] = (x[a] * pre) * (x[b] * pre) * inv_sqrt2;
}

/* [BASED s2] linear attention written as masked pairwise weights, with the
 * Taylor kernel in closed form (never forms phi).  Normaliser: the sum of
 * the same weights plus eps ([BASED App. D.4 "State size": denominator). */
void oracle_la_quadratic(const double *q, const double *k, const double *v,
                         int BH, int L, int d, int dv, double eps, double *y) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        const double *qh = q + (size_t)h * L * d;
        const double *kh = k + (size_t)h * L * d;
        const double *vh = v + (size_t)h * L * dv;
        double *yh = y + (size_t)h * L * dv;
        double *num = (double *)malloc(sizeof(double) * dv);
        for (int i = 0; i < L; ++i) {
            double den = 0.0;
            for (int c = 0; c < dv; ++c) num[c] = 0.0;
            for (int j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += qh[(size_t)i * d + e] * kh[(size_t)j * d + e];
                const double s = dot * inv_sqrt_d;
                const double a = 1.0 + s + 0.5 * s * s;
                den += a;
                for (int c = 0; c < dv; ++c) num[c] += a * vh[(size_t)j * dv + c];
            }
            for (int c = 0; c < dv; ++c) yh[(size_t)i * dv + c] = num[c] / (den + eps);
        }
        free(num);
    }
}

/* One token of the recurrent form on one head: update the state with
 * (k_t, v_t), then read it out with q_t.  [BASED s2]: constant-memory,
 * O(1)-per-token generation; [GSA App. A]: S += phi(k) v^T; [BASED App. D.4]:
 * the K-state z gives the denominator. */
static void recurrent_token(const double *qt, const double *kt, const double *vt,
                            int d, int dv, double eps, double *S, double *z,
                            double *yt, double *phiq, double *phik) {
    const int F = oracle_num_features(d);
    oracle_taylor_features(kt, d, phik);
    oracle_taylor_features(qt, d, phiq);
    for (int f = 0; f < F; ++f) {
        z[f] += phik[f];
        double *Sf = S + (size_t)f * dv;
        for (int c = 0; c < dv; ++c) Sf[c] += phik[f] * vt[c];
    }
    if (!yt) return;
    double den = 0.0;
    for (int f = 0; f < F; ++f) den += phiq[f] * z[f];
    for (int c = 0; c < dv; ++c) {
        double num = 0.0;
        for (int f = 0; f < F; ++f) num += phiq[f] * S[(size_t)f * dv + c];
        yt[c] = num / (den + eps);
    }
}

void oracle_la_recurrent(const double *q, const double *k, const double *v,
                         int BH, int L, int d, int dv, double eps,
                         const double *S_init, const double *z_init,
                         double *y, double *S_out, double *z_out) {
    const int F = oracle_num_features(d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        double *S = (double *)calloc((size_t)F * dv, sizeof(double));
        double *z = (double *)calloc((size_t)F, sizeof(double));
        double *phiq = (double *)malloc(sizeof(double) * F);
        double *phik = (double *)malloc(sizeof(double) * F);
        if (S_init) memcpy(S, S_init + (size_t)h * F * dv, sizeof(double) * F * dv);
        if (z_init) memcpy(z, z_init + (size_t)h * F, sizeof(double) * F);
        for (int t = 0; t < L; ++t) {
            const size_t tok = (size_t)h * L + t;
            recurrent_token(q + tok * d, k + tok * d, v + tok * dv, d, dv, eps, S, z,
                            y ? y + tok * dv : NULL, phiq, phik);
        }
        if (S_out) memcpy(S_out + (size_t)h * F * dv, S, sizeof(double) * F * dv);
        if (z_out) memcpy(z_out + (size_t)h * F, z, sizeof(double) * F);
        free(S); free(z); free(phiq); free(phik);
    }
}

/* [BASED App. B "Next Token Prediction"]: the KV-state update plus readout
 * for one new token, in place on the caller's state. */
void oracle_decode_step(const double *q, const double *k, const double *v,
                        int BH, int d, int dv, double eps,
                        double *S, double *z, double *y) {
    const int F = oracle_num_features(d);
#pragma omp parallel for schedule(static)
    for (int h = 0; h < BH; ++h) {
        double *phiq = (double *)malloc(sizeof(double) * F);
        double *phik = (double *)malloc(sizeof(double) * F);
        recurrent_token(q + (size_t)h * d, k + (size_t)h * d, v + (size_t)h * dv, d, dv, eps,
                        S + (size_t)h * F * dv, z + (size_t)h * F, y + (size_t)h * dv, phiq, phik);
        free(phiq); free(phik);
    }
}

/* [BASED s4 "Local Exact Attention"]: exact softmax attention over the
 * preceding `window` keys (the query's own key included), causal. */
void oracle_swa(const double *q, const double *k, const double *v,
                int BH, int L, int dqk, int dv, int window, double scale,
                double *y) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        const double *qh = q + (size_t)h * L * dqk;
        const double *kh = k + (size_t)h * L * dqk;
        const double *vh = v + (size_t)h * L * dv;
        double *yh = y + (size_t)h * L * dv;
        double *logit = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        for (int i = 0; i < L; ++i) {
            const int j0 = i - window + 1 > 0 ? i - window + 1 : 0;
            const int n = i - j0 + 1;
            double m = -INFINITY;
            for (int jj = 0; jj < n; ++jj) {
                const int j = j0 + jj;
                double dot = 0.0;
                for (int e = 0; e < dqk; ++e) dot += qh[(size_t)i * dqk + e] * kh[(size_t)j * dqk + e];
                logit[jj] = scale * dot;
                if (logit[jj] > m) m = logit[jj];
            }
            double l = 0.0;
            for (int jj = 0; jj < n; ++jj) {
                logit[jj] = exp(logit[jj] - m);
                l += logit[jj];
            }
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int jj = 0; jj < n; ++jj) acc += logit[jj] * vh[(size_t)(j0 + jj) * dv + c];
                yh[(size_t)i * dv + c] = acc / l;
            }
        }
        free(logit);
    }
}

/* [BASED s4 "Local Exact Attention"]: the window keeps a w-sized key/value
 * cache.  Ring reading: the token at position p lives in slot p mod window,
 * so a prefix of L tokens leaves its last min(L, window) tokens in their
 * slots (other slots are left as they are). */
void oracle_swa_cache_fill(const double *k, const double *v, int BH, int L, int dqk, int dv,
                           int window, double *kc, double *vc) {
    for (int h = 0; h < BH; ++h) {
        const int p0 = L - window > 0 ? L - window : 0;
        for (int p = p0; p < L; ++p) {
            const int slot = p % window;
            for (int e = 0; e < dqk; ++e)
                kc[((size_t)h * window + slot) * dqk + e] = k[((size_t)h * L + p) * dqk + e];
            for (int c = 0; c < dv; ++c)
                vc[((size_t)h * window + slot) * dv + c] = v[((size_t)h * L + p) * dv + c];
        }
    }
}

/* One next-token step of the window for the token at position pos[h]: its
 * key and value go into slot pos mod window, then it attends with exact
 * softmax to positions max(0, pos-window+1) .. pos (its own included), each
 * read from its slot -- the same sum as oracle_swa's row pos. */
void oracle_swa_decode_step(const double *q, const double *k, const double *v,
                            const long long *pos, int BH, int dqk, int dv, int window,
                            double scale, double *kc, double *vc, double *y) {
    double *logit = (double *)malloc(sizeof(double) * (size_t)window);
    for (int h = 0; h < BH; ++h) {
        const long long p = pos[h];
        double *kh = kc + (size_t)h * window * dqk;
        double *vh = vc + (size_t)h * window * dv;
        const int slot = (int)(p % window);
        for (int e = 0; e < dqk; ++e) kh[(size_t)slot * dqk + e] = k[(size_t)h * dqk + e];
        for (int c = 0; c < dv; ++c) vh[(size_t)slot * dv + c] = v[(size_t)h * dv + c];
        const long long t0 = p - window + 1 > 0 ? p - window + 1 : 0;
        const int n = (int)(p - t0 + 1);
        double m = -INFINITY;
        for (int jj = 0; jj < n; ++jj) {
            const int s = (int)((t0 + jj) % window);
            double dot = 0.0;
            for (int e = 0; e < dqk; ++e) dot += q[(size_t)h * dqk + e] * kh[(size_t)s * dqk + e];
            logit[jj] = scale * dot;
            if (logit[jj] > m) m = logit[jj];
        }
        double l = 0.0;
        for (int jj = 0; jj < n; ++jj) {
            const double e = exp(logit[jj] - m);
            logit[jj] = e;
            l += e;
        }
        for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int jj = 0; jj < n; ++jj) acc += logit[jj] * vh[(size_t)((t0 + jj) % window) * dv + c];
            y[(size_t)h * dv + c] = acc / l;
        }
    }
    free(logit);
}

/* Gradients of the causal Taylor linear attention output for an upstream
 * gradient dy (training-mode prefill: [BASED s5] notes prefill also serves
 * training).  The chain rule through the closed form
 *   y_i = N_i / D_i,  N_i = sum_{j<=i} a_ij v_j,  D_i = sum_{j<=i} a_ij + eps,
 *   a_ij = 1 + s_ij + s_ij^2 / 2,  s_ij = q_i . k_j / sqrt(d):
 *   gN_i = dy_i / D_i,  gD_i = -(dy_i . y_i) / D_i,
 *   ga_ij = gN_i . v_j + gD_i,  gs_ij = ga_ij (1 + s_ij),
 *   dq_i = sum_{j<=i} gs_ij k_j / sqrt(d),  dk_j = sum_{i>=j} gs_ij q_i / sqrt(d),
 *   dv_j = sum_{i>=j} a_ij gN_i.
 * O(L^2) per head; q,k [BH,L,d], v,dy [BH,L,dv]. */
void oracle_la_backward(const double *q, const double *k, const double *v, const double *dy,
                        int BH, int L, int d, int dv, double eps,
                        double *dq, double *dk, double *dv_out) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        const double *qh = q + (size_t)h * L * d;
        const double *kh = k + (size_t)h * L * d;
        const double *vh = v + (size_t)h * L * dv;
        const double *dyh = dy + (size_t)h * L * dv;
        double *dqh = dq + (size_t)h * L * d;
        double *dkh = dk + (size_t)h * L * d;
        double *dvh = dv_out + (size_t)h * L * dv;
        double *gN = (double *)malloc(sizeof(double) * (size_t)L * dv);
        double *gD = (double *)malloc(sizeof(double) * (size_t)L);
        double *num = (double *)malloc(sizeof(double) * dv);
        for (int i = 0; i < L; ++i) {  /* forward values and the gradients of N_i, D_i */
            double Di = eps;
            for (int c = 0; c < dv; ++c) num[c] = 0.0;
            for (int j = 0; j < i + 1; ++j) {  /* keys up to and including i */
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += qh[(size_t)i * d + e] * kh[(size_t)j * d + e];
                const double sij = dot * inv_sqrt_d;
                const double aij = 1.0 + sij + 0.5 * sij * sij;
                Di += aij;
                for (int c = 0; c < dv; ++c) num[c] += aij * vh[(size_t)j * dv + c];
            }
            double dy_dot_y = 0.0;
            for (int c = 0; c < dv; ++c) {
                gN[(size_t)i * dv + c] = dyh[(size_t)i * dv + c] / Di;
                dy_dot_y += dyh[(size_t)i * dv + c] * (num[c] / Di);
            }
            gD[i] = -dy_dot_y / Di;
        }
        for (size_t e = 0; e < (size_t)L * d; ++e) dqh[e] = dkh[e] = 0.0;
        for (size_t e = 0; e < (size_t)L * dv; ++e) dvh[e] = 0.0;
        for (int i = 0; i < L; ++i) {
            for (int j = i; j >= 0; --j) {  /* the same keys, any order */
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += qh[(size_t)i * d + e] * kh[(size_t)j * d + e];
                const double sij = dot * inv_sqrt_d;
                const double aij = 1.0 + sij + 0.5 * sij * sij;
                double ga = gD[i];
                for (int c = 0; c < dv; ++c) ga += gN[(size_t)i * dv + c] * vh[(size_t)j * dv + c];
                const double gs = ga * (1.0 + sij) * inv_sqrt_d;
                for (int e = 0; e < d; ++e) {
                    dqh[(size_t)i * d + e] += gs * kh[(size_t)j * d + e];
                    dkh[(size_t)j * d + e] += gs * qh[(size_t)i * d + e];
                }
                for (int c = 0; c < dv; ++c) dvh[(size_t)j * dv + c] += aij * gN[(size_t)i * dv + c];
            }
        }
        free(gN); free(gD); free(num);
    }
}

/* Gradients of the sliding-window softmax output (oracle_swa) for an
 * upstream gradient dy ([BASED s4 "Local Exact Attention"]; training-mode
 * prefill, [BASED s5]).  With P_ij = exp(l_ij - m_i) / sum_j' exp(l_ij' - m_i)
 * over the window of query i and l_ij = scale q_i . k_j, the chain rule
 * through y_i = sum_j P_ij v_j gives
 *   dv_j = sum_i P_ij dy_i,   dP_ij = dy_i . v_j,   D_i = sum_j P_ij dP_ij,
 *   dl_ij = P_ij (dP_ij - D_i),
 *   dq_i = scale sum_j dl_ij k_j,   dk_j = scale sum_i dl_ij q_i.
 * q,k [BH,L,dqk], v,dy [BH,L,dv]. */
void oracle_swa_backward(const double *q, const double *k, const double *v, const double *dy,
                         int BH, int L, int dqk, int dv, int window, double scale,
                         double *dq, double *dk, double *dv_out) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        const double *qh = q + (size_t)h * L * dqk;
        const double *kh = k + (size_t)h * L * dqk;
        const double *vh = v + (size_t)h * L * dv;
        const double *dyh = dy + (size_t)h * L * dv;
        double *dqh = dq + (size_t)h * L * dqk;
        double *dkh = dk + (size_t)h * L * dqk;
        double *dvh = dv_out + (size_t)h * L * dv;
        double *p = (double *)malloc(sizeof(double) * (size_t)(window > 0 ? window : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(window > 0 ? window : 1));
        for (size_t e = 0; e < (size_t)L * dqk; ++e) dqh[e] = dkh[e] = 0.0;
        for (size_t e = 0; e < (size_t)L * dv; ++e) dvh[e] = 0.0;
        for (int i = 0; i < L; ++i) {
            const int j0 = i + 1 - window < 0 ? 0 : i + 1 - window;  /* first key in the window */
            const int n = i - j0 + 1;
            double m = -INFINITY;
            for (int jj = 0; jj < n; ++jj) {
                double dot = 0.0;
                for (int e = 0; e < dqk; ++e) dot += qh[(size_t)i * dqk + e] * kh[(size_t)(j0 + jj) * dqk + e];
                p[jj] = scale * dot;
                if (p[jj] > m) m = p[jj];
            }
            double l = 0.0;
            for (int jj = 0; jj < n; ++jj) {
                p[jj] = exp(p[jj] - m);
                l += p[jj];
            }
            double D = 0.0;
            for (int jj = 0; jj < n; ++jj) {
                p[jj] /= l;
                double dot = 0.0;
                for (int c = 0; c < dv; ++c) dot += dyh[(size_t)i * dv + c] * vh[(size_t)(j0 + jj) * dv + c];
                dp[jj] = dot;
                D += p[jj] * dot;
            }
            for (int jj = 0; jj < n; ++jj) {
                const int j = j0 + jj;
                const double dl = p[jj] * (dp[jj] - D) * scale;
                for (int e = 0; e < dqk; ++e) {
                    dqh[(size_t)i * dqk + e] += dl * kh[(size_t)j * dqk + e];
                    dkh[(size_t)j * dqk + e] += dl * qh[(size_t)i * dqk + e];
                }
                for (int c = 0; c < dv; ++c) dvh[(size_t)j * dv + c] += p[jj] * dyh[(size_t)i * dv + c];
            }
        }
        free(p);
        free(dp);
    }
}

/* J_phi(x)^T u: the gradient of sum_f u_f phi_f(x) with respect to the raw
 * vector x, for the feature map of oracle_taylor_features (x~ = x d^(-1/4);
 * d phi_lin[a] / dx_c = pre [a == c]; d phi_quad[a][b] / dx_c =
 * pre ([a == c] x~_b + [b == c] x~_a) / sqrt(2)). */
static void taylor_jacobian_t(const double *x, int d, const double *u, double *out) {
    const double pre = 1.0 / sqrt(sqrt((double)d));
    const double inv_sqrt2 = 1.0 / sqrt(2.0);
    for (int c = 0; c < d; ++c) {
        double acc = u[1 + c];
        for (int b = 0; b < d; ++b)
            acc += (u[1 + d + c * d + b] + u[1 + d + b * d + c]) * (x[b] * pre) * inv_sqrt2;
        out[c] = acc * pre;
    }
}

/* The same gradients as oracle_la_backward, by the recurrent (feature) form:
 * the chain rule through y_i = phi(q_i)^T S_i / (phi(q_i).z_i + eps) with
 * S_i = sum_{j<=i} phi(k_j) v_j^T, z_i = sum_{j<=i} phi(k_j):
 *   forward over i:  g_i = dy_i / D_i,  h_i = -(dy_i . y_i) / D_i,
 *                    dq_i = J_phi(q_i)^T (S_i g_i + h_i z_i);
 *   backward over j: R_j = sum_{i>=j} phi(q_i) g_i^T,  r_j = sum_{i>=j} phi(q_i) h_i,
 *                    dk_j = J_phi(k_j)^T (R_j v_j + r_j),  dv_j = R_j^T phi(k_j).
 * O(L F dv) per head. */
void oracle_la_backward_recurrent(const double *q, const double *k, const double *v, const double *dy,
                                  int BH, int L, int d, int dv, double eps,
                                  double *dq, double *dk, double *dv_out) {
    const int F = oracle_num_features(d);
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < BH; ++h) {
        const double *qh = q + (size_t)h * L * d;
        const double *kh = k + (size_t)h * L * d;
        const double *vh = v + (size_t)h * L * dv;
        const double *dyh = dy + (size_t)h * L * dv;
        double *dqh = dq + (size_t)h * L * d;
        double *dkh = dk + (size_t)h * L * d;
        double *dvh = dv_out + (size_t)h * L * dv;
        double *S = (double *)calloc((size_t)F * dv, sizeof(double));
        double *z = (double *)calloc((size_t)F, sizeof(double));
        double *phiq = (double *)malloc(sizeof(double) * F);
        double *phik = (double *)malloc(sizeof(double) * F);
        double *u = (double *)malloc(sizeof(double) * F);
        double *y = (double *)malloc(sizeof(double) * dv);
        double *gN = (double *)malloc(sizeof(double) * (size_t)L * dv);
        double *gD = (double *)malloc(sizeof(double) * (size_t)L);
        for (int i = 0; i < L; ++i) {
            recurrent_token(qh + (size_t)i * d, kh + (size_t)i * d, vh + (size_t)i * dv, d, dv, eps, S, z, y,
                            phiq, phik);
            double den = eps;
            for (int f = 0; f < F; ++f) den += phiq[f] * z[f];
            double dy_dot_y = 0.0;
            for (int c = 0; c < dv; ++c) {
                gN[(size_t)i * dv + c] = dyh[(size_t)i * dv + c] / den;
                dy_dot_y += dyh[(size_t)i * dv + c] * y[c];
            }
            gD[i] = -dy_dot_y / den;
            for (int f = 0; f < F; ++f) {
                double acc = gD[i] * z[f];
                for (int c = 0; c < dv; ++c) acc += S[(size_t)f * dv + c] * gN[(size_t)i * dv + c];
                u[f] = acc;
            }
            taylor_jacobian_t(qh + (size_t)i * d, d, u, dqh + (size_t)i * d);
        }
        /* reverse sweep: S and z now hold R and r */
        memset(S, 0, sizeof(double) * (size_t)F * dv);
        memset(z, 0, sizeof(double) * (size_t)F);
        for (int j = L - 1; j >= 0; --j) {
            oracle_taylor_features(qh + (size_t)j * d, d, phiq);
            for (int f = 0; f < F; ++f) {
                z[f] += phiq[f] * gD[j];
                for (int c = 0; c < dv; ++c) S[(size_t)f * dv + c] += phiq[f] * gN[(size_t)j * dv + c];
            }
            oracle_taylor_features(kh + (size_t)j * d, d, phik);
            for (int f = 0; f < F; ++f) {
                double acc = z[f];
                for (int c = 0; c < dv; ++c) acc += S[(size_t)f * dv + c] * vh[(size_t)j * dv + c];
                u[f] = acc;
            }
            taylor_jacobian_t(kh + (size_t)j * d, d, u, dkh + (size_t)j * d);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < F; ++f) acc += phik[f] * S[(size_t)f * dv + c];
                dvh[(size_t)j * dv + c] = acc;
            }
        }
        free(S); free(z); free(phiq); free(phik); free(u); free(y); free(gN); free(gD);
    }
}
