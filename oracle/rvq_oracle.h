/*
 * rvq_oracle.h -- plain CPU reference of the routed RVQ-MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this code; only the tests, the benchmark's CPU-baseline leg and the
 * smoke check do.  It shares no code, header, table or helper with the GPU
 * path.
 *
 * All arithmetic is IEEE double, written out in the order the definitions
 * state; every weight is reconstructed explicitly as c1 + c2 + c3 (the matrix
 * is materialised row by row, the opposite of the fast method, on purpose).
 *
 * Sources (the pages this follows):
 *   [FR] "Exécuter Kimi K3 avec 29 Go de RAM à 0,50 tok/s" (fr.news.hada.io,
 *        topic 32035) -- sections "Quantification et exactitude",
 *        "Architecture de streaming depuis le disque", "Lecture anticipée et
 *        prédiction du routeur", "Budget RAM et fenêtre de performance étroite".
 *   [RU] "WASTE: запускаем полную Kimi K3 на MacBook Pro с 64 ГБ памяти"
 *        (feed.hirify.me) -- section "Расчёт строится на устройстве MoE".
 *
 * Layouts (canonical, shared with the inputs the tests generate):
 *   codebook of one expert : [3 matrices: gate, up, down][3 stages][256][8],
 *                            fp32 (dtype 0) or IEEE fp16 bits (dtype 1)
 *   record of one expert   : gate [F][d/8][3] u8, up [F][d/8][3] u8,
 *                            down [d][F/8][3] u8 (one byte per stage)
 *   router                 : W_r [d][E] fp32 row-major
 */
#ifndef RVQ_ORACLE_H
#define RVQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RVQO_STAGES 3
#define RVQO_CODES 256
#define RVQO_VEC 8

/* Threads the row loops use (OpenMP max threads; 1 without OpenMP). */
int rvq_oracle_threads(void);
/* Set the OpenMP thread count of later calls (n >= 1; no effect without OpenMP).
 * Results do not depend on it (rows are summed sequentially). */
void rvq_oracle_set_threads(int n);

/* IEEE binary16 bit pattern -> double, by field decoding. */
double rvq_oracle_half_to_double(uint16_t h);

/* x_i = h_i / sqrt(sum_i h_i^2 / d + eps).  Returns 0, or -1 on bad args. */
int rvq_oracle_rmsnorm(int d, const float *h, double eps, double *x_out);

/* logits[e] = sum_{i ascending} x[i] * W_r[i][e], in double. */
int rvq_oracle_router(int d, int n_experts, const double *x, const float *w_r, double *logits);

/* Top-k by a full sort on (logit descending, id ascending); gates are the
 * softmax over the k selected logits.  margin = l_(k) - l_(k+1) (or +inf when
 * k == E); min_gap = smallest difference between consecutive selected logits
 * (+inf when k == 1). */
int rvq_oracle_topk(int n_experts, int k, const double *logits, int32_t *ids, double *gates,
                    double *margin, double *min_gap);

/* out[r] = sum_s sum_i (C0[c0][i] + C1[c1][i] + C2[c2][i]) * v[8s + i] for one
 * RVQ matrix of shape [rows][cols]; codes [rows][cols/8][3]; codebook
 * [3][256][8] of dtype cb_dtype. */
int rvq_oracle_matvec(int rows, int cols, const void *codebook, int cb_dtype, const uint8_t *codes,
                      const double *v, double *out);

/* One expert's SwiGLU FFN: a = W_g x, b = W_u x, h = silu(a) * b, y = W_d h.
 * Any of pre_gate/pre_up/h_out may be NULL. */
int rvq_oracle_expert(int d, int ffn, const void *codebook, int cb_dtype, const uint8_t *record,
                      const double *x, double *pre_gate, double *pre_up, double *h_out, double *y);

/* Gate-weighted combine of k already-selected experts:
 * out[q] = sum_{j ascending} gates[j] * y_j[q]  (+ resid[q] if resid != NULL).
 * codebooks[j] / records[j] are expert ids[j]'s data. */
int rvq_oracle_moe(int d, int ffn, int k, const double *gates, const void *const *codebooks,
                   int cb_dtype, const uint8_t *const *records, const double *x, const float *resid,
                   double *out);

/* CRC-32 of n bytes, one bit at a time: the remainder of the polynomial
 * division that defines the checksum (generator x^32 + x^26 + x^23 + x^22 +
 * x^16 + x^12 + x^11 + x^10 + x^8 + x^7 + x^5 + x^4 + x^2 + x + 1, bits
 * taken least significant first, register preset to all ones and inverted
 * at the end).  [FR] "Architecture de streaming depuis le disque": an expert
 * record's payload may be checked by its crc32. */
uint32_t rvq_oracle_crc32(const uint8_t *p, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
