/* Runs the fp64 serial oracle (oracle/hla_serial.c, linked in, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer) on inputs read from a
 * file and writes its outputs and states to another, so that the test can
 * compare them with the ordinary build of the same oracle.
 *
 * Input file: long BH, H, n, d, dv; then q, k ([BH][n][d] fp32), v
 * ([BH][n][dv] fp32), gamma ([H] fp64), state_in (HLA-2 then AHLA layout,
 * fp64).  Output file: for each of the eight (family, ratio, decay) cases the
 * output [BH][n][dv] and the final state, fp64. */
#include <stdio.h>
#include <stdlib.h>

int oracle_hla2(const float *q, const float *k, const float *v, double *o, long BH, long H, long n,
                long d, long dv, const double *gamma, int ratio, const double *state_in,
                double *state_out, int threads);
int oracle_ahla(const float *q, const float *k, const float *v, double *o, long BH, long H, long n,
                long d, long dv, const double *gamma, int ratio, const double *state_in,
                double *state_out, int threads);

static void *read_all(FILE *f, size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short input\n"); exit(2); }
    return p;
}

int main(int argc, char **argv) {
    if (argc != 3) return 2;
    FILE *in = fopen(argv[1], "rb"), *out = fopen(argv[2], "wb");
    if (!in || !out) return 2;
    long dims[5];
    if (fread(dims, sizeof(long), 5, in) != 5) return 2;
    const long BH = dims[0], H = dims[1], n = dims[2], d = dims[3], dv = dims[4];
    float *q = read_all(in, sizeof(float) * BH * n * d);
    float *k = read_all(in, sizeof(float) * BH * n * d);
    float *v = read_all(in, sizeof(float) * BH * n * dv);
    double *g = read_all(in, sizeof(double) * H);
    const long s2 = d * d + d * dv + d, sa = 2 * d * dv + 2 * d;
    double *si2 = read_all(in, sizeof(double) * BH * s2);
    double *sia = read_all(in, sizeof(double) * BH * sa);
    double *o = malloc(sizeof(double) * BH * n * dv);
    double *so = malloc(sizeof(double) * BH * (s2 > sa ? s2 : sa));
    int rc = 0;
    for (int fam = 0; fam < 2; ++fam)
        for (int ratio = 0; ratio < 2; ++ratio)
            for (int decay = 0; decay < 2; ++decay) {
                const double *gp = decay ? g : NULL;
                if (fam == 0)
                    rc |= oracle_hla2(q, k, v, o, BH, H, n, d, dv, gp, ratio, si2, so, 1);
                else
                    rc |= oracle_ahla(q, k, v, o, BH, H, n, d, dv, gp, ratio, sia, so, 1);
                fwrite(o, sizeof(double), BH * n * dv, out);
                fwrite(so, sizeof(double), BH * (fam == 0 ? s2 : sa), out);
            }
    fclose(out);
    free(q); free(k); free(v); free(g); free(si2); free(sia); free(o); free(so);
    return rc;
}
