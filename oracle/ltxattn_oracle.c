/*
 * ltxattn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, double-precision CPU attention: the checker that the HIP
 * kernels are compared against.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or helper with the GPU library.
 *
 * What it computes (the softmax attention softmax(Q K^T / sqrt(D)) V that
 * every one of the four per-block attentions of the LTX-2 joint video+audio
 * DiT performs; the pairing of query and key/value streams is named in
 * TensorRT-LLM PR #16228 "LTX-2: replicate audio stream across Ulysses ranks
 * by default", section "Description"):
 *
 *   for every batch b, head h and query row i < Sq:
 *     s_j  = (sum_d q[b,i,h,d] * k[b,j,h,d]) / sqrt(D)      for j < kv_len
 *     m    = max_j s_j
 *     w_j  = exp(s_j - m)
 *     l    = sum_j w_j
 *     o[b,i,h,e] = (sum_j w_j * v[b,j,h,e]) / l
 *     lse  = m + log(l)                       (log-sum-exp, optional output)
 *
 * Keys j >= kv_len are padding (the audio stream is padded, PR #16228
 * "Description") and take no part: they are not read at all.  Padded query
 * rows are computed like any other row.
 *
 * Gated attention (named among the DiT's parts by TensorRT-Model-Connect PR
 * #1586, the commit onboarding LTX-2.5, without a formula): with a gate g of
 * the output's shape, already activated by the caller, the output is
 * g[b,i,h,e] * o[b,i,h,e].
 *
 * The QK-norm + rotary prologue (ltxattn_oracle_qk_prologue below): the
 * same commit keeps the network in bf16 with fp32 islands for norms and
 * RoPE, and its context-parallel DiT gathers keys after they are normed and
 * rotated; the pages give neither formula, so the reading is stated there.
 *
 * Inputs are float32 arrays holding bf16 values (exact), widened to double
 * here; layout [B, S, H, D] with D contiguous.  exp and log are libm's.
 * Work is split over threads by flat (b, h, i) row index; each row is
 * computed by one thread start to finish, so the result does not depend on
 * the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const float *q, *k, *v;
    const float *gate;     /* NULL, or [B,Sq,H,D]: multiplies the output elementwise */
    int64_t B, Sq, Sk, kv_len, H, D;
    const int64_t *rows;   /* NULL: all rows; else nrows (b, h, i) triples */
    int64_t nrows;
    double *out;           /* [B,Sq,H,D] when rows == NULL, else [nrows, D] */
    double *lse;           /* [B,Sq,H] or [nrows]; may be NULL */
    int64_t begin, end;    /* flat row range of this worker */
    int status;
} job_t;

/* One query row: the definition above, term by term. */
static int attend_row(const job_t *J, int64_t b, int64_t h, int64_t i,
                      double *o, double *lse_out)
{
    const int64_t H = J->H, D = J->D, L = J->kv_len;
    const double scale = 1.0 / sqrt((double)D);
    const float *qi = J->q + ((b * J->Sq + i) * H + h) * D;
    double *s = (double *)malloc((size_t)L * sizeof(double));
    if (!s) return -1;

    double m = -INFINITY;
    for (int64_t j = 0; j < L; ++j) {
        const float *kj = J->k + ((b * J->Sk + j) * H + h) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kj[d];
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        s[j] = exp(s[j] - m);   /* now the unnormalised weight w_j */
        l += s[j];
    }
    for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        const float *vj = J->v + ((b * J->Sk + j) * H + h) * D;
        for (int64_t e = 0; e < D; ++e) o[e] += s[j] * (double)vj[e];
    }
    for (int64_t e = 0; e < D; ++e) o[e] /= l;
    if (J->gate) {
        const float *gi = J->gate + ((b * J->Sq + i) * H + h) * D;
        for (int64_t e = 0; e < D; ++e) o[e] *= (double)gi[e];
    }
    if (lse_out) *lse_out = m + log(l);
    free(s);
    return 0;
}

static void *worker(void *arg)
{
    job_t *J = (job_t *)arg;
    for (int64_t r = J->begin; r < J->end; ++r) {
        int64_t b, h, i;
        double *o, *lse;
        if (J->rows) {
            b = J->rows[3 * r + 0];
            h = J->rows[3 * r + 1];
            i = J->rows[3 * r + 2];
            o = J->out + r * J->D;
            lse = J->lse ? J->lse + r : NULL;
        } else {
            /* flat index r enumerates (b, i, h) in memory order */
            h = r % J->H;
            i = (r / J->H) % J->Sq;
            b = r / (J->H * J->Sq);
            o = J->out + r * J->D;
            lse = J->lse ? J->lse + r : NULL;
        }
        if (attend_row(J, b, h, i, o, lse) != 0) { J->status = -1; return NULL; }
    }
    return NULL;
}

static int run(job_t *proto, int64_t nrows, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    pthread_t tid[256];
    job_t jobs[256];
    int64_t chunk = (nrows + nthreads - 1) / nthreads;
    int started = 0, status = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].begin = t * chunk < nrows ? t * chunk : nrows;
        jobs[t].end = (t + 1) * chunk < nrows ? (t + 1) * chunk : nrows;
        jobs[t].status = 0;
    }
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &jobs[t]) != 0) { status = -1; break; }
        started = t;
    }
    worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    for (int t = 0; t < nthreads; ++t) if (jobs[t].status) status = -1;
    return status;
}

static int check_sizes(int64_t B, int64_t Sq, int64_t Sk, int64_t kv_len, int64_t H, int64_t D)
{
    if (B < 1 || Sq < 0 || Sk < 1 || H < 1 || D < 1) return -2;
    if (kv_len < 1 || kv_len > Sk) return -2;
    return 0;
}

/* Full attention over all rows.  gate: NULL or [B,Sq,H,D]; out: [B,Sq,H,D]
 * double; lse: [B,Sq,H] (of the ungated softmax) or NULL.
 * Returns 0, -1 on allocation failure, -2 on bad sizes. */
int ltxattn_oracle_attention(const float *q, const float *k, const float *v, const float *gate,
                             int64_t B, int64_t Sq, int64_t Sk, int64_t kv_len,
                             int64_t H, int64_t D, double *out, double *lse,
                             int nthreads)
{
    int rc = check_sizes(B, Sq, Sk, kv_len, H, D);
    if (rc) return rc;
    job_t J = {q, k, v, gate, B, Sq, Sk, kv_len, H, D, NULL, 0, out, lse, 0, 0, 0};
    return run(&J, B * Sq * H, nthreads);
}

/* Selected rows only.  rows: nrows triples (b, h, i); out: [nrows, D];
 * lse: [nrows] or NULL. */
int ltxattn_oracle_attention_rows(const float *q, const float *k, const float *v, const float *gate,
                                  int64_t B, int64_t Sq, int64_t Sk, int64_t kv_len,
                                  int64_t H, int64_t D, const int64_t *rows,
                                  int64_t nrows, double *out, double *lse,
                                  int nthreads)
{
    int rc = check_sizes(B, Sq, Sk, kv_len, H, D);
    if (rc) return rc;
    for (int64_t r = 0; r < nrows; ++r) {
        if (rows[3 * r] < 0 || rows[3 * r] >= B || rows[3 * r + 1] < 0 ||
            rows[3 * r + 1] >= H || rows[3 * r + 2] < 0 || rows[3 * r + 2] >= Sq)
            return -2;
    }
    job_t J = {q, k, v, gate, B, Sq, Sk, kv_len, H, D, rows, nrows, out, lse, 0, 0, 0};
    return run(&J, nrows, nthreads);
}

/* ------------------------------------------------ QK-norm + rotary prologue
 *
 * Reading (the pages name the steps, not their formulas): an RMS norm over
 * the D channels of each (token, head) row with a learned per-channel
 * weight w[D] shared by all heads, then a rotation of channel pairs by
 * angles the caller tabulates per token position (the RoPE tables are data
 * baked into the DiT plan, PR #1586 "The DiT plan serves both grids"):
 *
 *   r   = 1 / sqrt((1/D) sum_d x_d^2 + eps)
 *   y_d = x_d * r * w_d
 *   pair i < D/2 = channels (a, c) = (i, i + D/2)  [pairing 0, rotate-half]
 *                                  or (2i, 2i + 1) [pairing 1, interleaved]
 *   z_a = y_a cos[s][i] - y_c sin[s][i]
 *   z_c = y_a sin[s][i] + y_c cos[s][i]
 *
 * computed in double; the result is the bf16 tensor the attention reads
 * (round to nearest, ties to even, straight from double), or z itself. */

/* The bf16 value nearest to v (ties to even), as its bit pattern. */
static uint16_t bf16_rne(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int ex;
    frexp(v, &ex);                       /* |v| = m 2^ex, m in [0.5, 1) */
    int e = ex - 1;                      /* floor(log2 |v|) */
    if (e < -126) e = -126;              /* below: bf16's subnormal spacing */
    const double ulp = ldexp(1.0, e - 7);
    const double r = nearbyint(v / ulp) * ulp;   /* default rounding mode: to nearest even */
    const float f = (float)r;            /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

int ltxattn_oracle_qk_prologue(const float *x, int64_t B, int64_t S, int64_t H, int64_t D,
                               const float *w, const float *cos_t, const float *sin_t,
                               double eps, int pairing, double *out, uint16_t *out_bf16)
{
    if (B < 1 || S < 1 || H < 1 || D < 2 || D % 2 || eps < 0 || (pairing != 0 && pairing != 1))
        return -2;
    const int64_t P = D / 2;
    double *y = (double *)malloc((size_t)D * sizeof(double));
    if (!y) return -1;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t h = 0; h < H; ++h) {
                const int64_t row = ((b * S + s) * H + h) * D;
                const float *xr = x + row;
                double ss = 0.0;
                for (int64_t d = 0; d < D; ++d) ss += (double)xr[d] * (double)xr[d];
                const double r = 1.0 / sqrt(ss / (double)D + eps);
                for (int64_t d = 0; d < D; ++d) y[d] = (double)xr[d] * r * (double)w[d];
                for (int64_t i = 0; i < P; ++i) {
                    const int64_t a = pairing == 0 ? i : 2 * i;
                    const int64_t c = pairing == 0 ? i + P : 2 * i + 1;
                    const double cs = (double)cos_t[s * P + i], sn = (double)sin_t[s * P + i];
                    const double za = y[a] * cs - y[c] * sn;
                    const double zc = y[a] * sn + y[c] * cs;
                    if (out) { out[row + a] = za; out[row + c] = zc; }
                    if (out_bf16) { out_bf16[row + a] = bf16_rne(za); out_bf16[row + c] = bf16_rne(zc); }
                }
            }
    free(y);
    return 0;
}
