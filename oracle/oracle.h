/* SLQ CPU oracle -- TEST INFRASTRUCTURE ONLY (see oracle.c for sources). */
#ifndef SLQ_ORACLE_H
#define SLQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oracle_num_threads(void);
void oracle_set_threads(int n);
void oracle_quantize(const float *W, int64_t n, int64_t k, int bits, int group,
                     int symmetric, uint8_t *q, float *scales, uint8_t *zeros);
void oracle_pack(const uint8_t *q, int64_t n, int64_t k, int bits, uint32_t *words);
void oracle_unpack(const uint32_t *words, int64_t n, int64_t k, int bits, uint8_t *q);
void oracle_dequantize(const uint8_t *q, const float *scales, const uint8_t *zeros,
                       int64_t n, int64_t k, int group, float *w_hat);
void oracle_gemm(const uint16_t *x, int64_t m, int64_t k, const float *w_hat, int64_t n,
                 double *y, double *bound);
void oracle_gemm_pairs(const uint16_t *x, int64_t k, const float *w_hat_rows,
                       const int64_t *xi, const int64_t *wi, int64_t npairs,
                       double *y, double *bound);
void oracle_row_lse(const float *a, int64_t rows, int64_t vocab, double *lse);
void oracle_ear_kl(const float *a, const float *b, int64_t rows, int64_t vocab,
                   double *ear, double *kl, double *means);
void oracle_ear_kl_topk(const float *a, const float *b, int64_t rows, int64_t vocab, int64_t K,
                        double T, double *ear, double *kl, double *means);
void oracle_quant_error(const float *W, const float *w_hat, const float *scales,
                        int64_t n, int64_t k, int group, double *out);
double oracle_bits_per_param(int bits, int meta_bits, int group);
double oracle_f16_value(uint16_t bits);
uint16_t oracle_f16_round_up(float s);
int oracle_compact_zero_bits(int bits);
void oracle_quantize_compact(const float *W, int64_t n, int64_t k, int bits, int group,
                             int symmetric, uint8_t *q, uint16_t *scales16, uint8_t *zeros);
int64_t oracle_pack_zeros(const uint8_t *zeros, int64_t count, int bits, uint8_t *out);
void oracle_dequantize_compact(const uint8_t *q, const uint16_t *scales16, const uint8_t *zpacked,
                               int64_t n, int64_t k, int group, int bits, float *w_hat);
void oracle_gptq_columns(const float *W, const float *U, const uint8_t *dead, int64_t n,
                         int64_t k, int bits, int group, uint8_t *q, float *scales,
                         uint8_t *zeros);
int oracle_mckp_search(int64_t L, int nb, const int64_t *sizes, const double *costs, int64_t W,
                       double tau, int32_t *choice, int64_t *budget_out, int64_t *size_out,
                       double *cost_out, double *best_out);

#ifdef __cplusplus
}
#endif
#endif
