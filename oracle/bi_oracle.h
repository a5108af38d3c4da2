/*
 * bi_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * Private to oracle/: the product library never includes this header.
 * All arrays are host memory, row-major, bf16 passed as raw uint16_t bits.
 * Functions return 0 on success, -1 on a bad shape, -2 on allocation failure.
 */
#ifndef BI_ORACLE_H
#define BI_ORACLE_H
#include <stdint.h>

uint16_t or_f32_to_bf16(float f);
float or_bf16_value(uint16_t b);
float or_fold_f32(const float *v, int64_t n);

int or_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, float *y32,
            int64_t M, int64_t N, int64_t K);
int or_gemm_exact(const uint16_t *x, const uint16_t *w, double *y,
                  int64_t M, int64_t N, int64_t K);
int or_gemm_absdot(const uint16_t *x, const uint16_t *w, double *a,
                   int64_t M, int64_t N, int64_t K);

int or_rmsnorm(const uint16_t *x, const uint16_t *g, uint16_t *y, float *rinv,
               int64_t M, int64_t H, float eps);
int or_rmsnorm_exact(const uint16_t *x, const uint16_t *g, double *y,
                     int64_t M, int64_t H, double eps);

int or_paged_decode_attn(const uint16_t *q, const uint16_t *kv,
                         const int32_t *block_table, const int32_t *ctx_lens,
                         uint16_t *out, int64_t B, int Hq, int Hkv, int D,
                         int PS, int64_t max_blocks, float scale);
int or_paged_decode_attn_exact(const uint16_t *q, const uint16_t *kv,
                               const int32_t *block_table,
                               const int32_t *ctx_lens, double *out, int64_t B,
                               int Hq, int Hkv, int D, int PS,
                               int64_t max_blocks, double scale);

/* bi_oracle_layer.c: element-wise steps of the decoder layer */
int or_rope_table(double theta, int D, int64_t max_pos, float *cos_t, float *sin_t);
int or_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, int64_t M, int heads,
            int D, int64_t x_stride, const float *cos_t, const float *sin_t,
            int64_t max_pos);
int or_silu_mul(const uint16_t *gu, uint16_t *y, int64_t M, int64_t F);
int or_add(const uint16_t *a, const uint16_t *b, uint16_t *y, int64_t n);

/* bi_oracle_sample.c: per-request counter-based sampling */
void or_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]);
float or_sample_uniform(uint64_t seed, uint64_t step, int64_t v);
int or_sample(const uint16_t *logits, int64_t M, int64_t V, const uint64_t *seeds,
              const uint64_t *steps, const float *temps, int32_t *tokens, float *best_score,
              float *second_score);
#endif
