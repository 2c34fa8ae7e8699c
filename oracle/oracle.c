/*
 * Plain fp64 CPU oracle for multi-head scaled dot-product attention (forward
 * and backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded input generator.
 *
 * Every function is the textbook definition written out in loops, in double
 * precision, with no blocking, no fusion and no skipping of masked work:
 *
 *   Q = Xq Wq^T + bq,  K = Xkv Wk^T + bk,  V = Xkv Wv^T + bv
 *       (four d_model x d_model linear layers, stored [out, in] as a torch
 *        linear layer stores them; "Transformer" study notes, multi-head
 *        attention section: formula, parameter list and class code)
 *   head split: head hd owns features [hd*d_k, (hd+1)*d_k) of each row
 *       (same section: view to [B, L, h, d_k] then transpose to [B, h, L, d_k])
 *   s_ij = (q_i . k_j) / sqrt(d_k)          (The Annotated Transformer,
 *       "Attention" section; d_k is the per-head width of the query)
 *   the score of a masked pair is REPLACED by -1e9 after scaling (same
 *       section: the mask fills the scaled scores with that constant)
 *   p_i = softmax over the key axis, o_i = sum_j p_ij v_j   (same section)
 *   merge heads back to [B, L, h*d_v], then out = Ocat Wo^T + bo
 *       ("Transformer" study notes, multi-head attention: Concat(head_1..h) W^O)
 *
 * Masks.  A key j is allowed for query i of batch b when
 *   (valid_lens == NULL or j < len(b, i))  and  (!causal or j <= i),
 * where len(b, i) = valid_lens[b] for lengths per batch [B] and
 * valid_lens[b*Lq + i] for lengths per query [B, Lq].
 * The valid_lens rule is the d2l reading (d2l Transformer digest, multi-head
 * attention prerequisites: valid lengths are repeated over the heads, and no
 * query attends to padded keys; its masked softmax takes them either per
 * sequence or per query, and the decoder's training pass gives query i the
 * length i + 1); the causal rule is the lower-triangular
 * "subsequent mask" whose 5x5 print keeps the diagonal ("Transformer" study
 * notes, mask-generation section; The Annotated Transformer, decoder section).
 * The two masks are combined by logical AND.  One mask serves every head.
 *
 * Softmax is evaluated as exp(s_j - max_k s_k) / sum exp(s_k - max): the same
 * number as the plain quotient, written so that large logits cannot overflow.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MASK_FILL (-1e9)

/* Round a double to the nearest bfloat16 value (8-bit significand, fp32
 * exponent range), ties to even.  Used only by the optional "bf16 storage"
 * mode below; exposed for its own test against torch's conversion. */
double oracle_round_bf16_f64(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    double m = frexp(fabs(x), &e);          /* |x| = m * 2^e, m in [0.5, 1) */
    /* bf16 keeps 8 significant bits for normals (2^-126 <= |x|); below that
     * the spacing is fixed at 2^-133. */
    int bits = 8;
    if (e - 1 < -126) bits = 8 - (-126 - (e - 1));
    if (bits < 0) return copysign(0.0, x);
    double scaled = ldexp(m, bits);          /* in [2^(bits-1), 2^bits) */
    double fl = floor(scaled);
    double rem = scaled - fl;
    double r;
    if (rem > 0.5) r = fl + 1.0;
    else if (rem < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double y = ldexp(r, e - bits);
    if (y > 3.3895313892515355e38) y = INFINITY;  /* beyond the largest bf16 */
    return copysign(y, x);
}

/* y[m, n] = sum_c x[m, c] * w[n, c] + (b ? b[n] : 0), ascending c. */
void oracle_linear_f64(const double* x, const double* w, const double* b,
                       double* y, long M, int Din, int Dout)
{
    long m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int n = 0; n < Dout; ++n) {
            double acc = 0.0;
            for (int c = 0; c < Din; ++c) acc += x[m * Din + c] * w[(long)n * Din + c];
            y[m * Dout + n] = acc + (b ? b[n] : 0.0);
        }
    }
}

static int key_allowed(const int* valid_lens, int vl_per_query, int Lq, int causal, int b, int i, int j)
{
    if (vl_per_query) {
        if (valid_lens && !(j < valid_lens[(long)b * Lq + i])) return 0;
    } else {
        if (valid_lens && !(j < valid_lens[b])) return 0;
    }
    if (causal && j > i) return 0;
    return 1;
}

/* The scaled scores of one query row against every key, masked pairs
 * replaced by the fill. */
static void row_scores(const double* qi, const double* k, double* s, int Lq, int Lk, int dk,
                       const int* valid_lens, int vl_per_query, int causal, int b, int i)
{
    const double scale = 1.0 / sqrt((double)dk);
    for (int j = 0; j < Lk; ++j) {
        double dot = 0.0;
        for (int t = 0; t < dk; ++t) dot += qi[t] * k[(long)j * dk + t];
        s[j] = dot * scale;
        if (!key_allowed(valid_lens, vl_per_query, Lq, causal, b, i, j)) s[j] = ORACLE_MASK_FILL;
    }
}

/* One query row of one (batch, head): the attention definition, every key. */
static void attend_row(const double* qi, const double* k, const double* v,
                       double* oi, double* pi, double* s,
                       int Lq, int Lk, int dk, int dv,
                       const int* valid_lens, int vl_per_query, int causal, int b, int i)
{
    row_scores(qi, k, s, Lq, Lk, dk, valid_lens, vl_per_query, causal, b, i);
    double mx = s[0];
    for (int j = 1; j < Lk; ++j) if (s[j] > mx) mx = s[j];
    double den = 0.0;
    for (int j = 0; j < Lk; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
    for (int j = 0; j < Lk; ++j) s[j] /= den;
    for (int t = 0; t < dv; ++t) {
        double acc = 0.0;
        for (int j = 0; j < Lk; ++j) acc += s[j] * v[(long)j * dv + t];
        oi[t] = acc;
    }
    if (pi) memcpy(pi, s, sizeof(double) * (size_t)Lk);
}

/*
 * Scaled dot-product attention on already split heads.
 *   q [B, h, Lq, dk], k [B, h, Lk, dk], v [B, h, Lk, dv]   (contiguous)
 *   o [B, h, R, dv] and, if p != NULL, p [B, h, R, Lk], where the R rows are
 *   rows[0..n_rows) (query indices) or, when rows == NULL, all Lq queries.
 *   valid_lens: NULL, [B] (vl_per_query == 0) or [B, Lq] (vl_per_query == 1).
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_sdpa_f64(const double* q, const double* k, const double* v,
                    double* o, double* p,
                    int B, int h, int Lq, int Lk, int dk, int dv,
                    const int* valid_lens, int vl_per_query, int causal,
                    const int* rows, int n_rows)
{
    if (B < 0 || h <= 0 || Lq < 0 || Lk <= 0 || dk <= 0 || dv <= 0) return -1;
    const int R = rows ? n_rows : Lq;
    if (rows)
        for (int r = 0; r < R; ++r) if (rows[r] < 0 || rows[r] >= Lq) return -1;
    int bad = 0;
    long bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < (long)B * h; ++bh) {
        const int b = (int)(bh / h);
        double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!s) { bad = 1; continue; }
        const double* qb = q + bh * (long)Lq * dk;
        const double* kb = k + bh * (long)Lk * dk;
        const double* vb = v + bh * (long)Lk * dv;
        for (int r = 0; r < R; ++r) {
            const int i = rows ? rows[r] : r;
            attend_row(qb + (long)i * dk, kb, vb,
                       o + (bh * R + r) * (long)dv,
                       p ? p + (bh * R + r) * (long)Lk : NULL, s,
                       Lq, Lk, dk, dv, valid_lens, vl_per_query, causal, b, i);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * The log of the softmax normaliser of each query row: with s_ij the scaled
 * scores (masked pairs replaced by the fill; row_scores, as attend_row),
 *   lse_i = log sum_j exp(s_ij),
 * so that the weights are exp(s_ij - lse_i) (The Annotated Transformer,
 * "Attention" section: softmax over the key axis).  Written as
 * max_j s_ij + log sum_j exp(s_ij - max) so large logits cannot overflow.
 * A row whose keys are all masked has every score equal to the fill, so its
 * lse is the fill + log(Lk).
 *   q [B, h, Lq, dk], k [B, h, Lk, dk] (contiguous); lse [B, h, Lq] written.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_sdpa_lse_f64(const double* q, const double* k, double* lse,
                        int B, int h, int Lq, int Lk, int dk,
                        const int* valid_lens, int vl_per_query, int causal)
{
    if (B < 0 || h <= 0 || Lq < 0 || Lk <= 0 || dk <= 0) return -1;
    int bad = 0;
    long bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < (long)B * h; ++bh) {
        const int b = (int)(bh / h);
        double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!s) { bad = 1; continue; }
        const double* qb = q + bh * (long)Lq * dk;
        const double* kb = k + bh * (long)Lk * dk;
        for (int i = 0; i < Lq; ++i) {
            row_scores(qb + (long)i * dk, kb, s, Lq, Lk, dk, valid_lens, vl_per_query, causal, b, i);
            double mx = s[0];
            for (int j = 1; j < Lk; ++j) if (s[j] > mx) mx = s[j];
            double den = 0.0;
            for (int j = 0; j < Lk; ++j) den += exp(s[j] - mx);
            lse[bh * (long)Lq + i] = mx + log(den);
        }
        free(s);
    }
    return bad ? -1 : 0;
}

static void round_all(double* a, long n)
{
    for (long i = 0; i < n; ++i) a[i] = oracle_round_bf16_f64(a[i]);
}

/*
 * Multi-head attention forward.
 *   xq [B, Lq, D], xkv [B, Lk, D]; w_* [D, D] stored [out, in]; b_* [D] or NULL.
 *   out [B, R, D] for the R query rows selected as in oracle_sdpa_f64.
 *   h heads of width dk = D / h (D must be a multiple of h).
 *   bf16_stages != 0: Q, K, V and the merged head output are rounded to the
 *   nearest bfloat16 before the next step reads them (the storage precision a
 *   bf16 pipeline gives those intermediates); 0 keeps everything in fp64.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_mha_f64(const double* xq, const double* xkv,
                   const double* w_q, const double* b_q,
                   const double* w_k, const double* b_k,
                   const double* w_v, const double* b_v,
                   const double* w_o, const double* b_o,
                   double* out, int B, int Lq, int Lk, int D, int h,
                   const int* valid_lens, int vl_per_query, int causal,
                   const int* rows, int n_rows, int bf16_stages)
{
    if (B < 0 || Lq < 0 || Lk <= 0 || D <= 0 || h <= 0 || D % h != 0) return -1;
    const int dk = D / h;
    const int R = rows ? n_rows : Lq;
    if (rows)
        for (int r = 0; r < R; ++r) if (rows[r] < 0 || rows[r] >= Lq) return -1;
    if (B == 0 || R == 0) return 0;

    /* Gather the selected query rows of X_q, then project. */
    double* xsel = (double*)malloc(sizeof(double) * (size_t)B * R * D);
    double* Qf = (double*)malloc(sizeof(double) * (size_t)B * R * D);
    double* Kf = (double*)malloc(sizeof(double) * (size_t)B * Lk * D);
    double* Vf = (double*)malloc(sizeof(double) * (size_t)B * Lk * D);
    double* qh = (double*)malloc(sizeof(double) * (size_t)B * R * D);
    double* kh = (double*)malloc(sizeof(double) * (size_t)B * Lk * D);
    double* vh = (double*)malloc(sizeof(double) * (size_t)B * Lk * D);
    double* oh = (double*)malloc(sizeof(double) * (size_t)B * R * D);
    double* ocat = (double*)malloc(sizeof(double) * (size_t)B * R * D);
    int rc = 0;
    if (!xsel || !Qf || !Kf || !Vf || !qh || !kh || !vh || !oh || !ocat) { rc = -1; goto done; }

    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r) {
            const int i = rows ? rows[r] : r;
            memcpy(xsel + ((long)b * R + r) * D, xq + ((long)b * Lq + i) * D, sizeof(double) * (size_t)D);
        }
    oracle_linear_f64(xsel, w_q, b_q, Qf, (long)B * R, D, D);
    oracle_linear_f64(xkv, w_k, b_k, Kf, (long)B * Lk, D, D);
    oracle_linear_f64(xkv, w_v, b_v, Vf, (long)B * Lk, D, D);
    if (bf16_stages) {
        round_all(Qf, (long)B * R * D);
        round_all(Kf, (long)B * Lk * D);
        round_all(Vf, (long)B * Lk * D);
    }

    /* Head split: [B, L, h, dk] -> [B, h, L, dk]. */
    for (int b = 0; b < B; ++b)
        for (int hd = 0; hd < h; ++hd) {
            for (int r = 0; r < R; ++r)
                for (int t = 0; t < dk; ++t)
                    qh[(((long)b * h + hd) * R + r) * dk + t] = Qf[((long)b * R + r) * D + hd * dk + t];
            for (int j = 0; j < Lk; ++j)
                for (int t = 0; t < dk; ++t) {
                    kh[(((long)b * h + hd) * Lk + j) * dk + t] = Kf[((long)b * Lk + j) * D + hd * dk + t];
                    vh[(((long)b * h + hd) * Lk + j) * dk + t] = Vf[((long)b * Lk + j) * D + hd * dk + t];
                }
        }

    /* Attention per head.  The query rows were already gathered, but the
     * causal rule needs each row's original index, so attend row by row with
     * that index. */
    {
        long bh;
        int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
        for (bh = 0; bh < (long)B * h; ++bh) {
            const int b = (int)(bh / h);
            double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
            if (!s) { bad = 1; continue; }
            for (int r = 0; r < R; ++r) {
                const int i = rows ? rows[r] : r;
                attend_row(qh + (bh * R + r) * (long)dk, kh + bh * (long)Lk * dk,
                           vh + bh * (long)Lk * dk, oh + (bh * R + r) * (long)dk, NULL, s,
                           Lq, Lk, dk, dk, valid_lens, vl_per_query, causal, b, i);
            }
            free(s);
        }
        if (bad) { rc = -1; goto done; }
    }

    /* Head merge: [B, h, R, dk] -> [B, R, h*dk]. */
    for (int b = 0; b < B; ++b)
        for (int hd = 0; hd < h; ++hd)
            for (int r = 0; r < R; ++r)
                for (int t = 0; t < dk; ++t)
                    ocat[((long)b * R + r) * D + hd * dk + t] = oh[(((long)b * h + hd) * R + r) * dk + t];
    if (bf16_stages) round_all(ocat, (long)B * R * D);

    oracle_linear_f64(ocat, w_o, b_o, out, (long)B * R, D, D);

done:
    free(xsel); free(Qf); free(Kf); free(Vf);
    free(qh); free(kh); free(vh); free(oh); free(ocat);
    return rc;
}

/*
 * Gradients of the attention above (the backward pass the pages' training
 * loops take through it: The Annotated Transformer and the d2l digest train
 * these models end to end).  For one (batch, head), with tau = 1/sqrt(dk),
 * p_i = softmax of row i as in attend_row and a loss whose gradient with
 * respect to o is do:
 *   dv_j  = sum_i p_ij do_i
 *   dp_ij = do_i . v_j
 *   ds_ij = p_ij (dp_ij - sum_l p_il dp_il)          (softmax Jacobian)
 *   dq_i  = tau sum_j ds_ij k_j,   dk_j = tau sum_i ds_ij q_i
 * where a masked score is the constant fill, so ds_ij of a masked pair does
 * not reach q or k (its p_ij is 0 anyway unless the whole row is masked).
 *   q, k, v, do as for oracle_sdpa_f64 (do shaped like o, all Lq rows);
 *   dq [B, h, Lq, dk], dk [B, h, Lk, dk], dv [B, h, Lk, dv] are written.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_sdpa_backward_f64(const double* q, const double* k, const double* v, const double* dout,
                             double* dq, double* dk, double* dv,
                             int B, int h, int Lq, int Lk, int dk_, int dv_,
                             const int* valid_lens, int vl_per_query, int causal)
{
    if (B < 0 || h <= 0 || Lq < 0 || Lk <= 0 || dk_ <= 0 || dv_ <= 0) return -1;
    const double tau = 1.0 / sqrt((double)dk_);
    int bad = 0;
    long bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < (long)B * h; ++bh) {
        const int b = (int)(bh / h);
        double* p = (double*)malloc(sizeof(double) * (size_t)Lk);
        double* s = (double*)malloc(sizeof(double) * (size_t)Lk);
        double* o = (double*)malloc(sizeof(double) * (size_t)dv_);
        double* dp = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!p || !s || !o || !dp) { bad = 1; free(p); free(s); free(o); free(dp); continue; }
        const double* qb = q + bh * (long)Lq * dk_;
        const double* kb = k + bh * (long)Lk * dk_;
        const double* vb = v + bh * (long)Lk * dv_;
        const double* gb = dout + bh * (long)Lq * dv_;
        double* dqb = dq + bh * (long)Lq * dk_;
        double* dkb = dk + bh * (long)Lk * dk_;
        double* dvb = dv + bh * (long)Lk * dv_;
        for (long x = 0; x < (long)Lq * dk_; ++x) dqb[x] = 0.0;
        for (long x = 0; x < (long)Lk * dk_; ++x) dkb[x] = 0.0;
        for (long x = 0; x < (long)Lk * dv_; ++x) dvb[x] = 0.0;
        for (int i = 0; i < Lq; ++i) {
            const double* qi = qb + (long)i * dk_;
            const double* gi = gb + (long)i * dv_;
            /* the forward row: weights p_i */
            attend_row(qi, kb, vb, o, p, s, Lq, Lk, dk_, dv_, valid_lens, vl_per_query, causal, b, i);
            double rowsum = 0.0;
            for (int j = 0; j < Lk; ++j) {
                double acc = 0.0;
                for (int t = 0; t < dv_; ++t) acc += gi[t] * vb[(long)j * dv_ + t];
                dp[j] = acc;
                rowsum += p[j] * dp[j];
            }
            for (int j = 0; j < Lk; ++j) {
                for (int t = 0; t < dv_; ++t) dvb[(long)j * dv_ + t] += p[j] * gi[t];
                if (!key_allowed(valid_lens, vl_per_query, Lq, causal, b, i, j)) continue;
                const double ds = p[j] * (dp[j] - rowsum);
                for (int t = 0; t < dk_; ++t) {
                    dqb[(long)i * dk_ + t] += tau * ds * kb[(long)j * dk_ + t];
                    dkb[(long)j * dk_ + t] += tau * ds * qi[t];
                }
            }
        }
        free(p); free(s); free(o); free(dp);
    }
    return bad ? -1 : 0;
}

/*
 * Gradients of one linear layer y = x W^T + b (W [Dout, Din] stored [out,
 * in]) for the output gradient dy [M, Dout], by the chain rule on
 * y[m, n] = sum_c x[m, c] W[n, c] + b[n]:
 *   dx[m, c] (+)= sum_n dy[m, n] W[n, c]     (added to dx when accumulate)
 *   dW[n, c]    = sum_m dy[m, n] x[m, c]
 *   db[n]       = sum_m dy[m, n]             (when db is not NULL)
 */
static void linear_backward(const double* dy, const double* x, const double* w,
                            double* dx, double* dw, double* db, long M, int Din, int Dout, int accumulate)
{
    /* Each sum runs over its index in ascending order; the loops visit the
     * operands row by row (the per-element order of additions is that of
     * the formulas above). */
    long m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double* row = dx + m * Din;
        double acc[Din];
        for (int c = 0; c < Din; ++c) acc[c] = 0.0;
        for (int n = 0; n < Dout; ++n) {
            const double a = dy[m * Dout + n];
            for (int c = 0; c < Din; ++c) acc[c] += a * w[(long)n * Din + c];
        }
        for (int c = 0; c < Din; ++c) row[c] = (accumulate ? row[c] : 0.0) + acc[c];
    }
    int n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < Dout; ++n) {
        double* wrow = dw + (long)n * Din;
        for (int c = 0; c < Din; ++c) wrow[c] = 0.0;
        double bsum = 0.0;
        for (long r = 0; r < M; ++r) {
            const double a = dy[r * Dout + n];
            for (int c = 0; c < Din; ++c) wrow[c] += a * x[r * Din + c];
            bsum += a;
        }
        if (db) db[n] = bsum;
    }
}

/* [B, L, h*dk] rows <-> [B, h, L, dk] heads: head hd owns features
 * [hd*dk, (hd+1)*dk) of each row (the split of oracle_mha_f64); to_heads
 * selects the direction. */
static void head_permute(double* rows, double* heads, int B, int L, int h, int dk, int to_heads)
{
    for (int b = 0; b < B; ++b)
        for (int hd = 0; hd < h; ++hd)
            for (int l = 0; l < L; ++l)
                for (int t = 0; t < dk; ++t) {
                    double* r = rows + ((long)b * L + l) * h * dk + hd * dk + t;
                    double* e = heads + (((long)b * h + hd) * L + l) * dk + t;
                    if (to_heads) *e = *r;
                    else *r = *e;
                }
}

/*
 * Gradients of the multi-head layer of oracle_mha_f64 (all query rows) for an
 * output gradient dout [B, Lq, D]: the training pass the pages take through
 * it (The Annotated Transformer and the d2l digest train these models end to
 * end), by the chain rule through each forward step in reverse:
 *   out = Ocat Wo^T + bo        -> dOcat, dWo, dbo   (linear_backward)
 *   head merge                  -> split dOcat into heads
 *   attention per head          -> dq, dk, dv        (oracle_sdpa_backward_f64)
 *   head split                  -> merge dQ, dK, dV
 *   Q = Xq Wq^T + bq            -> dXq, dWq, dbq
 *   K = Xkv Wk^T + bk, V = ...  -> dXkv = dK Wk + dV Wv, dWk, dbk, dWv, dbv
 * dxq [B, Lq, D] is the gradient through the query projection and dxkv
 * [B, Lk, D] the gradient through the key and value projections; when one
 * tensor feeds both (self-attention) its gradient is their sum.  dw_* [D, D],
 * db_* [D] (db_* may be NULL).
 * bf16_stages != 0: as in oracle_mha_f64, Q, K, V and the merged heads are
 * rounded to bfloat16 where they are made, and so are the gradients of the
 * merged heads and of Q, K and V (the storage precision of a bf16 pipeline).
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_mha_backward_f64(const double* xq, const double* xkv,
                            const double* w_q, const double* b_q,
                            const double* w_k, const double* b_k,
                            const double* w_v, const double* b_v,
                            const double* w_o, const double* dout,
                            double* dxq, double* dxkv,
                            double* dw_q, double* db_q, double* dw_k, double* db_k,
                            double* dw_v, double* db_v, double* dw_o, double* db_o,
                            int B, int Lq, int Lk, int D, int h,
                            const int* valid_lens, int vl_per_query, int causal, int bf16_stages)
{
    if (B < 0 || Lq < 0 || Lk <= 0 || D <= 0 || h <= 0 || D % h != 0) return -1;
    const int dk = D / h;
    const long Mq = (long)B * Lq, Mk = (long)B * Lk;
    double* Qf = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* Kf = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* Vf = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* qh = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* kh = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* vh = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* oh = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* ocat = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* docat = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* doh = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* dqh = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* dkh = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* dvh = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* dQ = (double*)malloc(sizeof(double) * (size_t)(Mq * D + 1));
    double* dK = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    double* dV = (double*)malloc(sizeof(double) * (size_t)(Mk * D + 1));
    int rc = 0;
    if (!Qf || !Kf || !Vf || !qh || !kh || !vh || !oh || !ocat || !docat || !doh || !dqh || !dkh || !dvh ||
        !dQ || !dK || !dV) { rc = -1; goto done; }

    /* The forward, keeping what the backward reads. */
    oracle_linear_f64(xq, w_q, b_q, Qf, Mq, D, D);
    oracle_linear_f64(xkv, w_k, b_k, Kf, Mk, D, D);
    oracle_linear_f64(xkv, w_v, b_v, Vf, Mk, D, D);
    if (bf16_stages) {
        round_all(Qf, Mq * D);
        round_all(Kf, Mk * D);
        round_all(Vf, Mk * D);
    }
    head_permute(Qf, qh, B, Lq, h, dk, 1);
    head_permute(Kf, kh, B, Lk, h, dk, 1);
    head_permute(Vf, vh, B, Lk, h, dk, 1);
    {
        long bh;
        int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
        for (bh = 0; bh < (long)B * h; ++bh) {
            double* srow = (double*)malloc(sizeof(double) * (size_t)Lk);
            if (!srow) { bad = 1; continue; }
            for (int i = 0; i < Lq; ++i)
                attend_row(qh + (bh * Lq + i) * dk, kh + bh * Lk * dk, vh + bh * Lk * dk, oh + (bh * Lq + i) * dk,
                           NULL, srow, Lq, Lk, dk, dk, valid_lens, vl_per_query, causal, (int)(bh / h), i);
            free(srow);
        }
        if (bad) { rc = -1; goto done; }
    }
    head_permute(ocat, oh, B, Lq, h, dk, 0);
    if (bf16_stages) round_all(ocat, Mq * D);

    /* Output projection. */
    linear_backward(dout, ocat, w_o, docat, dw_o, db_o, Mq, D, D, 0);
    if (bf16_stages) round_all(docat, Mq * D);

    /* Attention, head by head. */
    head_permute(docat, doh, B, Lq, h, dk, 1);
    if (oracle_sdpa_backward_f64(qh, kh, vh, doh, dqh, dkh, dvh, B, h, Lq, Lk, dk, dk,
                                 valid_lens, vl_per_query, causal) != 0) { rc = -1; goto done; }
    head_permute(dQ, dqh, B, Lq, h, dk, 0);
    head_permute(dK, dkh, B, Lk, h, dk, 0);
    head_permute(dV, dvh, B, Lk, h, dk, 0);
    if (bf16_stages) {
        round_all(dQ, Mq * D);
        round_all(dK, Mk * D);
        round_all(dV, Mk * D);
    }

    /* Input projections: K and V both read xkv, so their input gradients add. */
    linear_backward(dQ, xq, w_q, dxq, dw_q, db_q, Mq, D, D, 0);
    linear_backward(dK, xkv, w_k, dxkv, dw_k, db_k, Mk, D, D, 0);
    linear_backward(dV, xkv, w_v, dxkv, dw_v, db_v, Mk, D, D, 1);

done:
    free(Qf); free(Kf); free(Vf); free(qh); free(kh); free(vh); free(oh); free(ocat);
    free(docat); free(doh); free(dqh); free(dkh); free(dvh); free(dQ); free(dK); free(dV);
    return rc;
}

/*
 * Layer normalisation of each row of x [M, D] (per-feature gain a and bias b,
 * NULL meaning 1 and 0).  The pages print two forms:
 *   kind 0 (The Annotated Transformer, LayerNorm class):
 *       a * (x - mean) / (std + eps) + b, std with Bessel's correction (n-1)
 *   kind 1 (the "Transformer" study notes' code, a torch LayerNorm layer):
 *       a * (x - mean) / sqrt(var + eps) + b, var without correction (n)
 */
void oracle_layer_norm_f64(const double* x, const double* a, const double* b, double* y,
                           long M, int D, int kind, double eps)
{
    long m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const double* xr = x + m * D;
        double mean = 0.0;
        for (int c = 0; c < D; ++c) mean += xr[c];
        mean /= D;
        double ss = 0.0;
        for (int c = 0; c < D; ++c) ss += (xr[c] - mean) * (xr[c] - mean);
        double den;
        if (kind == 0) den = sqrt(ss / (D - 1)) + eps;
        else den = sqrt(ss / D + eps);
        for (int c = 0; c < D; ++c)
            y[m * D + c] = (a ? a[c] : 1.0) * (xr[c] - mean) / den + (b ? b[c] : 0.0);
    }
}

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
