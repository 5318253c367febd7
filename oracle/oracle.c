/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the int8 MQA KV
 * attention path computes.  Nothing in the product library links, includes or
 * calls this file; only the tests, the smoke check and the bench's CPU
 * baseline use it.  It shares no code, header, table or constant with the GPU
 * path.
 *
 * Sources (the pages, cited by title and section):
 *  - "Como funciona a inferência de IA, explicando claramente" (Red Hat),
 *    section "Por que o cache KV existe": to produce the next token, the
 *    current token's query is compared with the key of every earlier token and
 *    the values are summed with those weights; the query is only needed for
 *    the current token while keys and values are needed for the whole history.
 *  - "Character.AI: inference optimization", section 03 "Model architecture",
 *    technique table: multi-query attention (one K/V head), hybrid attention
 *    with a horizon of 1024 for local layers, KV shared across layers.
 *  - same page, section 05 "Quantization and cost": int8 on the attention KV
 *    cache.
 * The pages give no formula constant and no quantisation scheme.  The plainest
 * reading used here: softmax(q k^T / sqrt(d)) v over keys dequantised as
 * scale * code, with a symmetric per-token int8 code and an fp32 scale
 * max|x| / 127.
 *
 * Precision: attention in fp64 throughout.  The quantiser is specified in
 * fp32 (the scale is an fp32 number and the code is decided by an fp32
 * division), so it is written in fp32 on purpose.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <omp.h>

/* ------------------------------------------------------------------------ */
/* Quantiser: symmetric per-token int8 with an fp32 scale.                   */
/*   a  = max_c |x_c|                 (exact in any order)                    */
/*   s  = a / 127                     (IEEE fp32 division, nearest-even)      */
/*   q_c = clamp(rint(x_c / s), -127, 127), x_c / s an fp32 IEEE division,   */
/*         rint rounding half to even;  a == 0  ->  s = 0 and every q_c = 0.  */
/* ------------------------------------------------------------------------ */
void oracle_quantize_rows(int64_t rows, int32_t d, const float *x,
                          int8_t *codes, float *scales)
{
    for (int64_t t = 0; t < rows; ++t) {
        const float *row = x + t * (int64_t)d;
        float a = 0.0f;
        for (int32_t c = 0; c < d; ++c) {
            float v = fabsf(row[c]);
            if (v > a) a = v;
        }
        volatile float s = a / 127.0f;   /* volatile: keep it a stored fp32 */
        float sv = s;
        scales[t] = sv;
        for (int32_t c = 0; c < d; ++c) {
            int8_t code = 0;
            if (a != 0.0f) {
                volatile float r = row[c] / sv;
                float n = nearbyintf(r); /* default mode: nearest, ties even */
                if (n > 127.0f) n = 127.0f;
                if (n < -127.0f) n = -127.0f;
                code = (int8_t)n;
            }
            codes[t * (int64_t)d + c] = code;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Dequantise: xhat = (double) s * (double) code.  A 24-bit by 8-bit product  */
/* fits in 53 bits, so this is exact.                                         */
/* ------------------------------------------------------------------------ */
void oracle_dequantize_rows(int64_t rows, int32_t d, const int8_t *codes,
                            const float *scales, double *out)
{
    for (int64_t t = 0; t < rows; ++t)
        for (int32_t c = 0; c < d; ++c)
            out[t * (int64_t)d + c] =
                (double)scales[t] * (double)codes[t * (int64_t)d + c];
}

/* ------------------------------------------------------------------------ */
/* Attention of one query row over a dequantised single-head KV history.      */
/*                                                                            */
/* Keys are stored for absolute positions key_start .. key_start+n_keys-1.    */
/* A query at absolute position p with window W attends positions             */
/*   [lo, p]  with  lo = max(0, p - W + 1) if W > 0, else lo = 0,             */
/* i.e. W keys including its own (W = 0: the whole history).                  */
/*   sigma_j = (sum_c q_c * khat_{j,c}) * softmax_scale                       */
/*   w_j     = exp(sigma_j - max_j sigma_j),  Z = sum_j w_j                   */
/*   out_c   = sum_j w_j * vhat_{j,c} / Z                                     */
/* Returns 0, or -1 if the attended range is not fully stored (the caller     */
/* passed a history that does not cover the window).                          */
/* ------------------------------------------------------------------------ */
static int attend_one(int32_t d, const double *q, int64_t p, int32_t window,
                      int64_t key_start, int64_t n_keys,
                      const int8_t *kc, const float *ks,
                      const int8_t *vc, const float *vs,
                      double softmax_scale, double *out)
{
    int64_t lo = 0;
    if (window > 0) {
        lo = p - (int64_t)window + 1;
        if (lo < 0) lo = 0;
    }
    int64_t hi = p + 1; /* exclusive */
    if (lo < key_start || hi > key_start + n_keys || hi <= lo) return -1;

    const int64_t n = hi - lo;
    double *sigma = (double *)malloc((size_t)n * sizeof(double));
    if (!sigma) return -2;

    /* scores: sigma_j = (q . khat_j) * softmax_scale */
    for (int64_t j = 0; j < n; ++j) {
        const int64_t r = lo + j - key_start;
        double dot = 0.0;
        for (int32_t c = 0; c < d; ++c) {
            double k = (double)ks[r] * (double)kc[r * (int64_t)d + c];
            dot += q[c] * k;
        }
        sigma[j] = dot * softmax_scale;
    }
    /* softmax with the maximum subtracted */
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (sigma[j] > m) m = sigma[j];
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        sigma[j] = exp(sigma[j] - m);
        z += sigma[j];
    }
    /* weighted sum of the dequantised values */
    for (int32_t c = 0; c < d; ++c) out[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const int64_t r = lo + j - key_start;
        for (int32_t c = 0; c < d; ++c) {
            double v = (double)vs[r] * (double)vc[r * (int64_t)d + c];
            out[c] += sigma[j] * v;
        }
    }
    for (int32_t c = 0; c < d; ++c) out[c] /= z;
    free(sigma);
    return 0;
}

/* Many query rows against one KV history (one slot of one sequence).  Rows   */
/* are independent; OpenMP spreads them over the host cores.  Returns the     */
/* number of rows whose attended range was not stored (0 on success).         */
int64_t oracle_attend(int64_t n_rows, int32_t d, const double *q,
                      const int64_t *pos, const int32_t *window,
                      int64_t key_start, int64_t n_keys,
                      const int8_t *kc, const float *ks,
                      const int8_t *vc, const float *vs,
                      double softmax_scale, double *out)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t r = 0; r < n_rows; ++r) {
        int rc = attend_one(d, q + r * (int64_t)d, pos[r], window[r], key_start,
                            n_keys, kc, ks, vc, vs, softmax_scale,
                            out + r * (int64_t)d);
        if (rc != 0) bad += 1;
    }
    return bad;
}

/* The per-token KV size formula of "Como funciona a inferência de IA",        */
/* section "Qual é o tamanho real do cache KV?":                              */
/*   2 x num_layers x num_kv_heads x head_dim x dtype_bytes                   */
int64_t oracle_kv_bytes_per_token(int64_t num_layers, int64_t num_kv_heads,
                                  int64_t head_dim, int64_t dtype_bytes)
{
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes;
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
