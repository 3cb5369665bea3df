/*
 * hla_serial.c -- fp64 serial-recurrence oracle for second-order Higher-order
 * Linear Attention (HLA-2) and its asymmetric variant (AHLA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Source: "Resumen Tecnico: Atencion Lineal de Orden Superior (HLA)"
 * (gist.science/es/paper/2510.27258):
 *   - section "1. HLA de Segundo Orden": the prefix moments S^K (sum of k k^T),
 *     C^QV (sum of q v^T) and m^Q (sum of q); the cross-summaries G and h that
 *     remove the future terms from the naive product S^K C^QV; the unnormalised
 *     output o_t = q_t^T (S^K_t C^QV_t - G_t); the ratio-normalised variant with
 *     a masked denominator built from the analogous summaries.
 *   - section "2. Atencion Lineal de Orden Superior Asimetrica (AHLA)": the
 *     streaming summaries P^KV, m^K, E and n.
 *   - section "Contribuciones Clave", item 2: masked operators with and without
 *     exponential decay.
 *
 * The page names the summaries but prints no update rule.  The rules below are
 * the unique ones for which the page's output formula equals the masked matrix
 * definition
 *     HLA-2: o = tril( tril(QK^T) tril(QK^T)^T ) V
 *     AHLA : o = tril(QK^T) tril(QK^T) V
 * (checked against brute force of that definition by the test suite).
 *
 * Decay reading: every prefix moment decays by gamma per token
 * (S <- g S + k k^T, C <- g C + q v^T, m <- g m + q) and G, h hold exactly the
 * key-after-value part of the decayed product, so the output formula is
 * unchanged and the pair (i, j) of a term in o_t carries weight
 * gamma^((t-i)+(t-j)).  gamma = 1 is the undecayed operator.
 * AHLA under the same reading: every summary decays by gamma per token
 * (P <- g P + k v^T, E <- g E + k y^T, m^K <- g m^K + k, n <- g n + ...), so
 * the term A[t,i] A[i,j] v_j of o_t carries weight gamma^(t-j).
 *
 * All arithmetic is fp64.  Inputs are fp32 arrays (bf16-rounded inputs are
 * exactly representable in fp32); every value is upcast before use.
 *
 * Layouts (row-major, contiguous):
 *   q, k : [BH][n][d]      v : [BH][n][dv]      o : [BH][n][dv]  (fp64)
 *   HLA-2 compact state per (b,h): [S (d*d) | W (d*dv) | u (d)]
 *          with W = S^K C^QV - G and u = S^K m^Q - h
 *   AHLA state per (b,h):          [P (d*dv) | E (d*dv) | mK (d) | nk (d)]
 * head index for gamma: h = bh % H.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* one (b,h) sequence of HLA-2 in the page's summary form */
static void hla2_head(const float *q, const float *k, const float *v, double *o,
                      long n, long d, long dv, double g, int ratio,
                      const double *st_in, double *st_out, double *work)
{
    double *S = work;            /* d x d   key moment S^K             */
    double *C = S + d * d;       /* d x dv  query-value moment C^QV    */
    double *G = C + d * dv;      /* d x dv  cross-summary G            */
    double *m = G + d * dv;      /* d       query mass m^Q             */
    double *h = m + d;           /* d       cross-summary h            */
    double *kt = h + d;          /* d       current key (fp64)         */
    double *qt = kt + d;         /* d       current query              */
    double *vt = qt + d;         /* dv      current value              */
    double *kC = vt + dv;        /* dv      k^T C_{t-1}                */
    double *qS = kC + dv;        /* d       q^T S_t                    */
    double *num = qS + d;        /* dv      numerator                  */
    long a, b, j, t;

    memset(S, 0, sizeof(double) * (size_t)(d * d + 2 * d * dv + 2 * d));
    if (st_in) {
        /* resume from the compact state (S, W, u): with C = 0 and m = 0 the
         * choice G = -W, h = -u gives S C - G = W and S m - h = u, and the
         * update rules below stay exact from any starting point. */
        const double *Win = st_in + d * d, *uin = Win + d * dv;
        memcpy(S, st_in, sizeof(double) * (size_t)(d * d));
        for (a = 0; a < d * dv; ++a) G[a] = -Win[a];
        for (a = 0; a < d; ++a) h[a] = -uin[a];
    }
    const double g2 = g * g;
    for (t = 0; t < n; ++t) {
        for (a = 0; a < d; ++a) { kt[a] = k[t * d + a]; qt[a] = q[t * d + a]; }
        for (j = 0; j < dv; ++j) vt[j] = v[t * dv + j];

        /* cross-summaries: the new key k_t meets every earlier query-value
         * pair, i.e. the previous C and m (terms with key index > value index) */
        double km = 0.0;
        for (j = 0; j < dv; ++j) kC[j] = 0.0;
        for (a = 0; a < d; ++a) {
            km += kt[a] * m[a];
            for (j = 0; j < dv; ++j) kC[j] += kt[a] * C[a * dv + j];
        }
        for (a = 0; a < d; ++a) {
            for (j = 0; j < dv; ++j) G[a * dv + j] = g2 * G[a * dv + j] + g * kt[a] * kC[j];
            h[a] = g2 * h[a] + g * kt[a] * km;
        }
        /* prefix moments */
        for (a = 0; a < d; ++a)
            for (b = 0; b < d; ++b) S[a * d + b] = g * S[a * d + b] + kt[a] * kt[b];
        for (a = 0; a < d; ++a) {
            for (j = 0; j < dv; ++j) C[a * dv + j] = g * C[a * dv + j] + qt[a] * vt[j];
            m[a] = g * m[a] + qt[a];
        }
        /* read-out: q^T (S C - G) and, for the ratio form, q^T (S m - h) */
        for (b = 0; b < d; ++b) {
            double s = 0.0;
            for (a = 0; a < d; ++a) s += qt[a] * S[a * d + b];
            qS[b] = s;
        }
        for (j = 0; j < dv; ++j) num[j] = 0.0;
        for (b = 0; b < d; ++b)
            for (j = 0; j < dv; ++j) num[j] += qS[b] * C[b * dv + j] - qt[b] * G[b * dv + j];
        if (ratio) {
            double den = 0.0;
            for (b = 0; b < d; ++b) den += qS[b] * m[b] - qt[b] * h[b];
            for (j = 0; j < dv; ++j) o[t * dv + j] = num[j] / den;
        } else {
            for (j = 0; j < dv; ++j) o[t * dv + j] = num[j];
        }
    }
    if (st_out) {
        double *Wout = st_out + d * d, *uout = Wout + d * dv;
        memcpy(st_out, S, sizeof(double) * (size_t)(d * d));
        for (a = 0; a < d; ++a) {
            for (j = 0; j < dv; ++j) {
                double s = 0.0;
                for (b = 0; b < d; ++b) s += S[a * d + b] * C[b * dv + j];
                Wout[a * dv + j] = s - G[a * dv + j];
            }
            double s = 0.0;
            for (b = 0; b < d; ++b) s += S[a * d + b] * m[b];
            uout[a] = s - h[a];
        }
    }
}

/* one (b,h) sequence of AHLA in the page's summary form */
static void ahla_head(const float *q, const float *k, const float *v, double *o,
                      long n, long d, long dv, double g, int ratio,
                      const double *st_in, double *st_out, double *work)
{
    double *P = work;            /* d x dv  P^KV = sum k v^T              */
    double *E = P + d * dv;      /* d x dv  E = sum k_i y_i^T             */
    double *mK = E + d * dv;     /* d       key mass m^K                  */
    double *nk = mK + d;         /* d       n = sum k_i (q_i . m^K_i)     */
    double *kt = nk + d, *qt = kt + d, *vt = qt + d, *y = vt + dv;
    long a, j, t;

    if (st_in) memcpy(P, st_in, sizeof(double) * (size_t)(2 * d * dv + 2 * d));
    else memset(P, 0, sizeof(double) * (size_t)(2 * d * dv + 2 * d));
    for (t = 0; t < n; ++t) {
        for (a = 0; a < d; ++a) { kt[a] = k[t * d + a]; qt[a] = q[t * d + a]; }
        for (j = 0; j < dv; ++j) vt[j] = v[t * dv + j];
        for (a = 0; a < d; ++a)
            for (j = 0; j < dv; ++j) P[a * dv + j] = g * P[a * dv + j] + kt[a] * vt[j];
        /* y_t = P_t^T q_t : first-order read-out routed through key index */
        for (j = 0; j < dv; ++j) y[j] = 0.0;
        for (a = 0; a < d; ++a)
            for (j = 0; j < dv; ++j) y[j] += qt[a] * P[a * dv + j];
        for (a = 0; a < d; ++a)
            for (j = 0; j < dv; ++j) E[a * dv + j] = g * E[a * dv + j] + kt[a] * y[j];
        double s = 0.0;
        for (a = 0; a < d; ++a) { mK[a] = g * mK[a] + kt[a]; }
        for (a = 0; a < d; ++a) s += qt[a] * mK[a];
        for (a = 0; a < d; ++a) nk[a] = g * nk[a] + kt[a] * s;
        for (j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (a = 0; a < d; ++a) acc += qt[a] * E[a * dv + j];
            o[t * dv + j] = acc;
        }
        if (ratio) {
            double den = 0.0;
            for (a = 0; a < d; ++a) den += qt[a] * nk[a];
            for (j = 0; j < dv; ++j) o[t * dv + j] /= den;
        }
    }
    if (st_out) memcpy(st_out, P, sizeof(double) * (size_t)(2 * d * dv + 2 * d));
}

static int bad_dims(long BH, long n, long d, long dv)
{
    return BH < 0 || n < 0 || d < 1 || dv < 1;
}

/* Returns 0 on success, 1 on bad arguments, 2 on allocation failure. */
int oracle_hla2(const float *q, const float *k, const float *v, double *o,
                long BH, long H, long n, long d, long dv,
                const double *gamma, int ratio,
                const double *state_in, double *state_out, int threads)
{
    if (bad_dims(BH, n, d, dv) || H < 1 || (n > 0 && (!q || !k || !v || !o))) return 1;
    const long st = d * d + d * dv + d;
    const long wsz = d * d + 2 * d * dv + 2 * d + 2 * d + dv + dv + d + dv;
    int rc = 0;
    long bh;
#ifdef _OPENMP
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) reduction(| : rc)
#endif
    for (bh = 0; bh < BH; ++bh) {
        double *work = (double *)malloc(sizeof(double) * (size_t)wsz);
        if (!work) { rc |= 2; continue; }
        const double g = gamma ? gamma[bh % H] : 1.0;
        hla2_head(q + bh * n * d, k + bh * n * d, v + bh * n * dv, o + bh * n * dv,
                  n, d, dv, g, ratio,
                  state_in ? state_in + bh * st : NULL,
                  state_out ? state_out + bh * st : NULL, work);
        free(work);
    }
    (void)threads;
    return rc;
}

int oracle_ahla(const float *q, const float *k, const float *v, double *o,
                long BH, long H, long n, long d, long dv,
                const double *gamma, int ratio,
                const double *state_in, double *state_out, int threads)
{
    if (bad_dims(BH, n, d, dv) || H < 1 || (n > 0 && (!q || !k || !v || !o))) return 1;
    const long st = 2 * d * dv + 2 * d;
    const long wsz = 2 * d * dv + 2 * d + 2 * d + 2 * dv;
    int rc = 0;
    long bh;
#ifdef _OPENMP
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads) reduction(| : rc)
#endif
    for (bh = 0; bh < BH; ++bh) {
        double *work = (double *)malloc(sizeof(double) * (size_t)wsz);
        if (!work) { rc |= 2; continue; }
        const double g = gamma ? gamma[bh % H] : 1.0;
        ahla_head(q + bh * n * d, k + bh * n * d, v + bh * n * dv, o + bh * n * dv,
                  n, d, dv, g, ratio,
                  state_in ? state_in + bh * st : NULL,
                  state_out ? state_out + bh * st : NULL, work);
        free(work);
    }
    (void)threads;
    return rc;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
