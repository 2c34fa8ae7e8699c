/* Driver for the sanitizer build of the oracle (tests/test_oracle_sanitized.py):
 * runs every oracle entry point on small inputs that reach its edge cases
 * (fully masked rows, lengths above Lk, lengths per query, causal, selected
 * rows, an empty batch, rejected arguments) so AddressSanitizer and
 * UndefinedBehaviorSanitizer see every indexing path.  Prints one checksum
 * per call; the test only needs the run to finish cleanly. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_round_bf16_f64(double x);
void oracle_linear_f64(const double* x, const double* w, const double* b, double* y, long M, int Din, int Dout);
int oracle_sdpa_f64(const double* q, const double* k, const double* v, double* o, double* p, int B, int h, int Lq,
                    int Lk, int dk, int dv, const int* valid_lens, int vl_per_query, int causal, const int* rows,
                    int n_rows);
int oracle_mha_f64(const double* xq, const double* xkv, const double* w_q, const double* b_q, const double* w_k,
                   const double* b_k, const double* w_v, const double* b_v, const double* w_o, const double* b_o,
                   double* out, int B, int Lq, int Lk, int D, int h, const int* valid_lens, int vl_per_query,
                   int causal, const int* rows, int n_rows, int bf16_stages);
int oracle_sdpa_backward_f64(const double* q, const double* k, const double* v, const double* dout, double* dq,
                             double* dk, double* dv, int B, int h, int Lq, int Lk, int dk_, int dv_,
                             const int* valid_lens, int vl_per_query, int causal);
void oracle_layer_norm_f64(const double* x, const double* a, const double* b, double* y, long M, int D, int kind,
                           double eps);
int oracle_mha_backward_f64(const double* xq, const double* xkv, const double* w_q, const double* b_q,
                            const double* w_k, const double* b_k, const double* w_v, const double* b_v,
                            const double* w_o, const double* dout, double* dxq, double* dxkv, double* dw_q,
                            double* db_q, double* dw_k, double* db_k, double* dw_v, double* db_v, double* dw_o,
                            double* db_o, int B, int Lq, int Lk, int D, int h, const int* valid_lens,
                            int vl_per_query, int causal, int bf16_stages);

static double* filled(long n, unsigned seed) {
    double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    unsigned s = seed * 2654435761u + 1u;
    for (long i = 0; i < n; ++i) {
        s = s * 1664525u + 1013904223u;
        a[i] = ((double)(s >> 8) / 16777216.0) * 2.0 - 1.0;
    }
    return a;
}

static double sum(const double* a, long n) {
    double t = 0.0;
    for (long i = 0; i < n; ++i) t += a[i];
    return t;
}

int main(void) {
    int rc = 0;
    const int B = 3, h = 2, Lq = 7, Lk = 9, d = 8, D = 16;
    double *q = filled((long)B * h * Lq * d, 1), *k = filled((long)B * h * Lk * d, 2), *v = filled((long)B * h * Lk * d, 3);
    double *g = filled((long)B * h * Lq * d, 4);
    double *o = filled((long)B * h * Lq * d, 5), *p = filled((long)B * h * Lq * Lk, 6);
    const int vl1[3] = {0, 4, 20};                     /* fully masked, partial, above Lk */
    int vl2[3 * 7];
    for (int i = 0; i < B * Lq; ++i) vl2[i] = (i * 5) % (Lk + 3) - 1;   /* -1 .. Lk+1 */
    const int rows[3] = {0, 3, 6};
    for (int causal = 0; causal < 2; ++causal) {
        const int lq = causal ? Lk : Lq;               /* causal needs a square problem */
        double* qq = causal ? filled((long)B * h * Lk * d, 7) : q;
        double* oo = filled((long)B * h * lq * d, 8);
        double* pp = filled((long)B * h * lq * Lk, 9);
        rc |= oracle_sdpa_f64(qq, k, v, oo, pp, B, h, lq, Lk, d, d, NULL, 0, causal, NULL, 0);
        rc |= oracle_sdpa_f64(qq, k, v, oo, pp, B, h, lq, Lk, d, d, vl1, 0, causal, NULL, 0);
        printf("sdpa causal=%d %.12f %.12f\n", causal, sum(oo, (long)B * h * lq * d), sum(pp, (long)B * h * lq * Lk));
        if (causal) { free(qq); }
        free(oo);
        free(pp);
    }
    rc |= oracle_sdpa_f64(q, k, v, o, p, B, h, Lq, Lk, d, d, vl2, 1, 0, NULL, 0);
    rc |= oracle_sdpa_f64(q, k, v, o, p, B, h, Lq, Lk, d, d, vl2, 1, 0, rows, 3);
    rc |= oracle_sdpa_f64(q, k, v, o, NULL, 0, h, Lq, Lk, d, d, NULL, 0, 0, NULL, 0);         /* empty batch */
    if (oracle_sdpa_f64(q, k, v, o, p, B, h, Lq, Lk, d, d, NULL, 0, 0, (const int[]){Lq}, 1) != -1) rc |= 1;
    printf("sdpa lengths per query %.12f\n", sum(o, (long)B * h * 3 * d));

    double *dq = filled((long)B * h * Lq * d, 10), *dk = filled((long)B * h * Lk * d, 11), *dv = filled((long)B * h * Lk * d, 12);
    rc |= oracle_sdpa_backward_f64(q, k, v, g, dq, dk, dv, B, h, Lq, Lk, d, d, vl1, 0, 0);
    rc |= oracle_sdpa_backward_f64(q, k, v, g, dq, dk, dv, B, h, Lq, Lk, d, d, vl2, 1, 0);
    printf("backward %.12f %.12f %.12f\n", sum(dq, (long)B * h * Lq * d), sum(dk, (long)B * h * Lk * d),
           sum(dv, (long)B * h * Lk * d));

    double *xq = filled((long)B * Lq * D, 13), *xkv = filled((long)B * Lk * D, 14);
    double* w[4];
    double* bias[4];
    for (int i = 0; i < 4; ++i) {
        w[i] = filled((long)D * D, 20 + i);
        bias[i] = filled(D, 30 + i);
    }
    double* out = filled((long)B * Lq * D, 15);
    rc |= oracle_mha_f64(xq, xkv, w[0], bias[0], w[1], bias[1], w[2], bias[2], w[3], bias[3], out, B, Lq, Lk, D, 2,
                         vl1, 0, 0, NULL, 0, 0);
    rc |= oracle_mha_f64(xq, xkv, w[0], NULL, w[1], NULL, w[2], NULL, w[3], NULL, out, B, Lq, Lk, D, 2, vl2, 1, 0,
                         rows, 3, 1);
    if (oracle_mha_f64(xq, xkv, w[0], NULL, w[1], NULL, w[2], NULL, w[3], NULL, out, B, Lq, Lk, 15, 2, NULL, 0, 0,
                       NULL, 0, 0) != -1)
        rc |= 1;                                       /* D not a multiple of h */
    printf("mha %.12f\n", sum(out, (long)B * 3 * D));

    {
        double* gout = filled((long)B * Lq * D, 17);
        double *dxq = filled((long)B * Lq * D, 18), *dxkv = filled((long)B * Lk * D, 19);
        double* dwb[8];
        for (int i = 0; i < 8; ++i) dwb[i] = filled(i < 4 ? (long)D * D : D, 40 + i);
        rc |= oracle_mha_backward_f64(xq, xkv, w[0], bias[0], w[1], bias[1], w[2], bias[2], w[3], gout, dxq, dxkv,
                                      dwb[0], dwb[4], dwb[1], dwb[5], dwb[2], dwb[6], dwb[3], dwb[7], B, Lq, Lk, D, 2,
                                      vl1, 0, 0, 1);
        rc |= oracle_mha_backward_f64(xq, xkv, w[0], NULL, w[1], NULL, w[2], NULL, w[3], gout, dxq, dxkv, dwb[0],
                                      NULL, dwb[1], NULL, dwb[2], NULL, dwb[3], NULL, B, Lq, Lk, D, 2, vl2, 1, 0, 0);
        rc |= oracle_mha_backward_f64(xq, xkv, w[0], NULL, w[1], NULL, w[2], NULL, w[3], gout, dxq, dxkv, dwb[0],
                                      dwb[4], dwb[1], dwb[5], dwb[2], dwb[6], dwb[3], dwb[7], B, 0, Lk, D, 2, NULL, 0,
                                      0, 0);                     /* no queries: zero weight gradients */
        if (oracle_mha_backward_f64(xq, xkv, w[0], NULL, w[1], NULL, w[2], NULL, w[3], gout, dxq, dxkv, dwb[0], NULL,
                                    dwb[1], NULL, dwb[2], NULL, dwb[3], NULL, B, Lq, Lk, 15, 2, NULL, 0, 0, 0) != -1)
            rc |= 1;                                   /* D not a multiple of h */
        printf("mha backward %.12f %.12f\n", sum(dxkv, (long)B * Lk * D), sum(dwb[0], (long)D * D));
        free(gout); free(dxq); free(dxkv);
        for (int i = 0; i < 8; ++i) free(dwb[i]);
    }

    double* y = filled((long)B * Lq * D, 16);
    oracle_layer_norm_f64(xq, w[0], bias[0], y, (long)B * Lq, D, 0, 1e-6);
    oracle_layer_norm_f64(xq, NULL, NULL, y, (long)B * Lq, D, 1, 1e-5);
    oracle_linear_f64(xq, w[0], NULL, y, (long)B * Lq, D, D);
    printf("layer norm / linear %.12f %.6f\n", sum(y, (long)B * Lq * D), oracle_round_bf16_f64(1.0 / 3.0));

    free(q); free(k); free(v); free(g); free(o); free(p); free(dq); free(dk); free(dv);
    free(xq); free(xkv); free(out); free(y);
    for (int i = 0; i < 4; ++i) { free(w[i]); free(bias[i]); }
    printf("rc %d\n", rc);
    return rc;
}
