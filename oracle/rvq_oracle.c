/*
 * rvq_oracle.c -- plain, slow, obviously correct CPU reference of the routed
 * RVQ-MoE decode layer.  TEST INFRASTRUCTURE ONLY: see rvq_oracle.h.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off [-fopenmp] -shared -fPIC
 * (no -ffast-math: every operation is evaluated exactly as written).  The
 * OpenMP pragma only splits independent output rows; every row is summed
 * sequentially, so results are bitwise identical for any thread count.
 *
 * What each function follows:
 *  - rvq_oracle_matvec: the weight format and the "partial dot product table"
 *    method of [FR] "Quantification et exactitude" (3-stage residual VQ,
 *    256-entry codebooks over 8-wide vectors, 3.00 bits per weight) and [RU]
 *    "Расчёт строится на устройстве MoE" (the matrix is never unfolded by the
 *    method).  The table method is exact in real arithmetic, so the oracle is
 *    the plain definition it shortcuts: rebuild every weight as the sum of its
 *    three stage vectors and take the dot product.  Reading: the 8 weights of
 *    a vector are consecutive entries of one output row along the reduction
 *    dimension; a weight is c1 + c2 + c3 with no scale or bias (none is
 *    stated).
 *  - rvq_oracle_expert: one expert = gate, up and down matrices stored
 *    contiguously ([FR] "Architecture de streaming depuis le disque"); the FFN
 *    form is not on the pages, the SwiGLU reading is taken:
 *    y = W_d (silu(W_g x) * (W_u x)), silu(z) = z / (1 + exp(-z)).
 *  - rvq_oracle_router / rvq_oracle_topk: the router picks 16 expert ids per
 *    token ([FR] "Lecture anticipée et prédiction du routeur", "Budget RAM et
 *    fenêtre de performance étroite").  The score function is not stated; the
 *    reading taken is top-k on raw logits then a softmax over the k selected,
 *    ties broken toward the lower id, ids emitted in descending logit order.
 *  - rvq_oracle_rmsnorm: RMS normalisation with unit weight before routing in
 *    the layer chain (a reading; the pages do not describe the trunk's norm).
 */
#include "rvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void rvq_oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int rvq_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

double rvq_oracle_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24); /* zero or subnormal: mant * 2^-24 */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(mant | 0x400), expo - 25); /* 1.mant * 2^(expo-15) */
    }
    return sign ? -v : v;
}

static double cb_value(const void *cb, int cb_dtype, size_t idx) {
    if (cb_dtype == 0) return (double)((const float *)cb)[idx];
    return rvq_oracle_half_to_double(((const uint16_t *)cb)[idx]);
}

int rvq_oracle_rmsnorm(int d, const float *h, double eps, double *x_out) {
    if (d <= 0 || !h || !x_out) return -1;
    double ss = 0.0;
    for (int i = 0; i < d; i++) ss += (double)h[i] * (double)h[i];
    double r = sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; i++) x_out[i] = (double)h[i] / r;
    return 0;
}

int rvq_oracle_router(int d, int n_experts, const double *x, const float *w_r, double *logits) {
    if (d <= 0 || n_experts <= 0 || !x || !w_r || !logits) return -1;
    for (int e = 0; e < n_experts; e++) {
        double acc = 0.0;
        for (int i = 0; i < d; i++) acc += x[i] * (double)w_r[(size_t)i * n_experts + e];
        logits[e] = acc;
    }
    return 0;
}

typedef struct {
    double logit;
    int32_t id;
} scored;

static int cmp_scored(const void *pa, const void *pb) {
    const scored *a = (const scored *)pa, *b = (const scored *)pb;
    if (a->logit > b->logit) return -1;
    if (a->logit < b->logit) return 1;
    return (a->id > b->id) - (a->id < b->id);
}

int rvq_oracle_topk(int n_experts, int k, const double *logits, int32_t *ids, double *gates,
                    double *margin, double *min_gap) {
    if (n_experts <= 0 || k <= 0 || k > n_experts || !logits || !ids || !gates) return -1;
    scored *s = (scored *)malloc(sizeof(scored) * (size_t)n_experts);
    if (!s) return -1;
    for (int e = 0; e < n_experts; e++) {
        s[e].logit = logits[e];
        s[e].id = e;
    }
    qsort(s, (size_t)n_experts, sizeof(scored), cmp_scored);
    double denom = 0.0;
    for (int j = 0; j < k; j++) {
        ids[j] = s[j].id;
        gates[j] = exp(s[j].logit - s[0].logit);
        denom += gates[j];
    }
    for (int j = 0; j < k; j++) gates[j] = gates[j] / denom;
    if (margin) *margin = (k < n_experts) ? s[k - 1].logit - s[k].logit : INFINITY;
    if (min_gap) {
        double g = INFINITY;
        for (int j = 0; j + 1 < k; j++) {
            double dd = s[j].logit - s[j + 1].logit;
            if (dd < g) g = dd;
        }
        *min_gap = g;
    }
    free(s);
    return 0;
}

int rvq_oracle_matvec(int rows, int cols, const void *codebook, int cb_dtype, const uint8_t *codes,
                      const double *v, double *out) {
    if (rows <= 0 || cols <= 0 || cols % RVQO_VEC || !codebook || !codes || !v || !out) return -1;
    if (cb_dtype != 0 && cb_dtype != 1) return -1;
    const int n_slices = cols / RVQO_VEC;
    const size_t stage_stride = (size_t)RVQO_CODES * RVQO_VEC;
    /* decode the three stage codebooks to double once (exact for fp32 and fp16) */
    double *cb = (double *)malloc(sizeof(double) * RVQO_STAGES * stage_stride);
    if (!cb) return -1;
    for (size_t idx = 0; idx < RVQO_STAGES * stage_stride; idx++) cb[idx] = cb_value(codebook, cb_dtype, idx);
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; r++) {
        double acc = 0.0;
        for (int j = 0; j < n_slices; j++) {
            const uint8_t *c = codes + ((size_t)r * n_slices + j) * RVQO_STAGES;
            const double *c1 = cb + 0 * stage_stride + (size_t)c[0] * RVQO_VEC;
            const double *c2 = cb + 1 * stage_stride + (size_t)c[1] * RVQO_VEC;
            const double *c3 = cb + 2 * stage_stride + (size_t)c[2] * RVQO_VEC;
            for (int i = 0; i < RVQO_VEC; i++) {
                double w = (c1[i] + c2[i]) + c3[i]; /* the explicit c1 + c2 + c3 reconstruction */
                acc += w * v[(size_t)j * RVQO_VEC + i];
            }
        }
        out[r] = acc;
    }
    free(cb);
    return 0;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

int rvq_oracle_expert(int d, int ffn, const void *codebook, int cb_dtype, const uint8_t *record,
                      const double *x, double *pre_gate, double *pre_up, double *h_out, double *y) {
    if (d <= 0 || ffn <= 0 || d % RVQO_VEC || ffn % RVQO_VEC || !codebook || !record || !x || !y)
        return -1;
    const size_t elem = cb_dtype == 0 ? 4 : 2;
    const size_t mat_cb = (size_t)RVQO_STAGES * RVQO_CODES * RVQO_VEC * elem;
    const size_t gate_bytes = (size_t)ffn * (d / RVQO_VEC) * RVQO_STAGES;
    const uint8_t *cb = (const uint8_t *)codebook;
    double *a = (double *)malloc(sizeof(double) * (size_t)ffn * 3);
    if (!a) return -1;
    double *b = a + ffn, *h = a + 2 * (size_t)ffn;
    int rc = rvq_oracle_matvec(ffn, d, cb + 0 * mat_cb, cb_dtype, record, x, a);
    if (!rc) rc = rvq_oracle_matvec(ffn, d, cb + 1 * mat_cb, cb_dtype, record + gate_bytes, x, b);
    if (!rc) {
        for (int r = 0; r < ffn; r++) h[r] = silu(a[r]) * b[r];
        rc = rvq_oracle_matvec(d, ffn, cb + 2 * mat_cb, cb_dtype, record + 2 * gate_bytes, h, y);
    }
    if (!rc) {
        if (pre_gate) memcpy(pre_gate, a, sizeof(double) * (size_t)ffn);
        if (pre_up) memcpy(pre_up, b, sizeof(double) * (size_t)ffn);
        if (h_out) memcpy(h_out, h, sizeof(double) * (size_t)ffn);
    }
    free(a);
    return rc;
}

int rvq_oracle_moe(int d, int ffn, int k, const double *gates, const void *const *codebooks,
                   int cb_dtype, const uint8_t *const *records, const double *x, const float *resid,
                   double *out) {
    if (d <= 0 || ffn <= 0 || k <= 0 || !gates || !codebooks || !records || !x || !out) return -1;
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    if (!y) return -1;
    for (int q = 0; q < d; q++) out[q] = 0.0;
    int rc = 0;
    for (int j = 0; j < k && !rc; j++) {
        rc = rvq_oracle_expert(d, ffn, codebooks[j], cb_dtype, records[j], x, NULL, NULL, NULL, y);
        if (!rc)
            for (int q = 0; q < d; q++) out[q] += gates[j] * y[q];
    }
    if (!rc && resid)
        for (int q = 0; q < d; q++) out[q] += (double)resid[q];
    free(y);
    return rc;
}

uint32_t rvq_oracle_crc32(const uint8_t *p, int64_t n) {
    /* the generator's coefficients x^0 .. x^31 as bits 31 .. 0 (x^32 implied) */
    const uint32_t gen = 0xEDB88320u;
    uint32_t r = 0xFFFFFFFFu;
    for (int64_t i = 0; i < n; i++) {
        r ^= (uint32_t)p[i];
        for (int b = 0; b < 8; b++) r = (r & 1u) ? (r >> 1) ^ gen : r >> 1;
    }
    return r ^ 0xFFFFFFFFu;
}
