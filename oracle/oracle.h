/*
 * oracle.h -- plain, slow, fp64 CPU reference for Taylor linear attention
 * (BASED) and causal sliding-window softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no source with the HIP
 * library.
 *
 * Sources (page title, then section):
 *   [BASED] "Simple linear attention language models balance the
 *           recall-throughput tradeoff" (arXiv 2402.18668v2 summary page):
 *           s2 "Preliminaries" (linear attention: exp(q.k) replaced by
 *           phi(q).phi(k), associativity, O(1)-per-token recurrent form);
 *           s4 "The BASED Architecture" ("Taylor Linear Attention": 2nd-order
 *           Taylor feature map, projected dim d' = 16; "Local Exact
 *           Attention": each query sees the preceding w keys);
 *           App. B "IO Aware Implementations" (prefill produces outputs and
 *           the cumulative state; next-token step updates the KV state);
 *           App. D.4 "State size" (an extra K-state gives the denominator).
 *   [GSA]   "Gated Slot Attention for Efficient Linear-Time Sequence
 *           Modeling" (arXiv 2409.07146v2 summary page), App. A "Linear
 *           Attention and its Chunkwise Form" (matrix-valued recurrent state
 *           updated by key-value outer products).
 *
 * Conventions shared by every routine
 *   - All arrays are dense, row-major, fp64.  "BH" is the number of
 *     independent (batch, head) pairs; every routine loops over them and
 *     treats them independently (OpenMP over BH).
 *   - q, k: [BH, L, d]   v: [BH, L, dv]   y: [BH, L, dv]
 *   - Taylor features: F = 1 + d + d*d.  For x~ = x * d^(-1/4):
 *       phi(x)[0]            = 1
 *       phi(x)[1 + a]        = x~_a                      (a = 0..d-1)
 *       phi(x)[1 + d + a*d+b] = x~_a * x~_b / sqrt(2)     (a-major)
 *     so that phi(q).phi(k) = 1 + s + s^2/2 with s = q.k / sqrt(d), the
 *     2nd-order Taylor polynomial of exp(s) [BASED s4].
 *   - State: S [BH, F, dv] and z [BH, F], rows in the feature order above.
 *
 * Parity pins for every routine are in tests/test_oracle_pins.py.
 */
#ifndef BASED_ORACLE_H
#define BASED_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Number of Taylor features for feature dim d: 1 + d + d*d. */
int oracle_num_features(int d);

/* phi(x) for one vector x[d] (raw, not pre-scaled) into out[F]. */
void oracle_taylor_features(const double *x, int d, double *out);

/* Causal Taylor linear attention, quadratic (parallel) form.  Never builds
 * features: uses the closed form a_ij = 1 + s_ij + s_ij^2/2 with
 * s_ij = q_i.k_j / sqrt(d), and y_i = sum_{j<=i} a_ij v_j /
 * (sum_{j<=i} a_ij + eps).  O(L^2) per head. */
void oracle_la_quadratic(const double *q, const double *k, const double *v,
                         int BH, int L, int d, int dv, double eps, double *y);

/* Causal Taylor linear attention, recurrent form, token by token with the
 * explicit F-wide features: S += phi(k_t) v_t^T, z += phi(k_t), then
 * y_t = phi(q_t)^T S / (phi(q_t).z + eps).  S_init/z_init may be NULL
 * (zero initial state).  S_out/z_out may be NULL; they receive the state
 * after the last token.  y may be NULL. */
void oracle_la_recurrent(const double *q, const double *k, const double *v,
                         int BH, int L, int d, int dv, double eps,
                         const double *S_init, const double *z_init,
                         double *y, double *S_out, double *z_out);

/* One next-token step, in place on S [BH,F,dv] and z [BH,F]:
 * update with (k, v) first, then read out with q (the current token is
 * included, as in the causal definition).  q,k: [BH,d]; v,y: [BH,dv]. */
void oracle_decode_step(const double *q, const double *k, const double *v,
                        int BH, int d, int dv, double eps,
                        double *S, double *z, double *y);

/* Causal sliding-window softmax attention by brute force.  Query i sees
 * keys j in [max(0, i-window+1), i] (window keys including itself):
 * y_i = sum_j e_ij v_j / sum_j e_ij, e_ij = exp(scale*q_i.k_j - m_i),
 * m_i = max_j scale*q_i.k_j over the same j.  q,k: [BH,L,dqk]. */
void oracle_swa(const double *q, const double *k, const double *v,
                int BH, int L, int dqk, int dv, int window, double scale,
                double *y);

/* The window's key/value cache (ring of `window` slots per head; the token
 * at position p lives in slot p mod window).  Fill from a prefix of L
 * tokens: slots of its last min(L, window) tokens are written, the others
 * are left untouched.  k: [BH,L,dqk]; kc: [BH,window,dqk]. */
void oracle_swa_cache_fill(const double *k, const double *v, int BH, int L, int dqk, int dv,
                           int window, double *kc, double *vc);

/* One next-token step of the window for head h at position pos[h] >= 0:
 * writes k, v into slot pos mod window, then y = exact softmax attention of
 * q over positions max(0, pos-window+1) .. pos read from their slots.
 * q,k: [BH,dqk]; v,y: [BH,dv]; kc/vc updated in place. */
void oracle_swa_decode_step(const double *q, const double *k, const double *v,
                            const long long *pos, int BH, int dqk, int dv, int window,
                            double scale, double *kc, double *vc, double *y);

/* Gradients of la_quadratic's output for an upstream gradient dy (chain
 * rule through the closed form; O(L^2) per head).  q,k,dq,dk [BH,L,d];
 * v,dy,dv [BH,L,dv]. */
void oracle_la_backward(const double *q, const double *k, const double *v, const double *dy,
                        int BH, int L, int d, int dv, double eps,
                        double *dq, double *dk, double *dv_out);

/* The same gradients by the recurrent (feature) form, O(L F dv) per head:
 * a forward sweep with S_i, z_i gives D_i, y_i, g_i = dy_i / D_i,
 * h_i = -(dy_i . y_i) / D_i and dq_i = J_phi(q_i)^T (S_i g_i + h_i z_i); a
 * backward sweep with R_j = sum_{i>=j} phi(q_i) g_i^T and
 * r_j = sum_{i>=j} phi(q_i) h_i gives dk_j = J_phi(k_j)^T (R_j v_j + r_j) and
 * dv_j = R_j^T phi(k_j).  Shapes as oracle_la_backward. */
void oracle_la_backward_recurrent(const double *q, const double *k, const double *v, const double *dy,
                                  int BH, int L, int d, int dv, double eps,
                                  double *dq, double *dk, double *dv_out);

/* Number of OpenMP threads the routines above use. */
int oracle_num_threads(void);

/* Gradients (dq, dk, dv) of oracle_swa for the upstream gradient dy, by the
 * chain rule through the window's softmax.  O(L w) per head. */
void oracle_swa_backward(const double *q, const double *k, const double *v, const double *dy,
                         int BH, int L, int dqk, int dv, int window, double scale,
                         double *dq, double *dk, double *dv_out);

#ifdef __cplusplus
}
#endif
#endif
