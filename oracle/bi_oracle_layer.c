/*
 * bi_oracle_layer.c -- plain CPU oracle for the element-wise steps of a
 * Llama-style decoder layer built around the batch-invariant kernels.
 *
 * TEST INFRASTRUCTURE ONLY, like bi_oracle.c: nothing in the product library
 * links, loads or calls this file, and it shares no code with the HIP path.
 *
 * Sources: the LLM-42 digest (problem statement: the whole forward of a
 * decoder, with its normalisation, projections and attention, has to give
 * the same bits for a token whether it is verified alone or in a group) and
 * the Determinism article (section 4: every reduction order fixed by the
 * data alone; section 5: no reduced-precision intermediates).  The pages name
 * the layer's steps only; the formulas below are the standard Llama ones,
 * with these readings (fp32 arithmetic, one bf16 rounding per step):
 *
 *   RoPE (rotate-half pairs i, i + D/2, i < D/2):
 *     a_i(p) = p * theta^(-2i/D), in double; c = (float)cos(a), s = (float)sin(a)
 *     y_i       = bf16( x_i * c - x_{i+D/2} * s )
 *     y_{i+D/2} = bf16( x_{i+D/2} * c + x_i * s )
 *     each product rounded to fp32, then the sum or difference (no FMA).
 *   SiLU-gated product of the up projection's two halves [gate | up]:
 *     y = bf16( (g / (1 + exp(-g))) * u ),  exp in fp32, four roundings.
 *   Residual add: y = bf16(a + b) with one fp32 addition.
 *
 * All arrays are host memory, row-major, bf16 passed as raw uint16_t bits.
 * Parity: RoPE (given the same table) and the residual add are bit-exact;
 * the SiLU product's exp is the platform's, so its last bits are unpinned
 * and covered by the tolerance.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "bi_oracle.h"

static float lay_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* cos/sin table [max_pos][D/2] for the RoPE reading above. */
int or_rope_table(double theta, int D, int64_t max_pos, float *cos_t, float *sin_t)
{
    if (D <= 0 || D % 2 != 0 || max_pos <= 0 || theta <= 0.0)
        return -1;
    const int half = D / 2;
    for (int64_t p = 0; p < max_pos; ++p) {
        for (int i = 0; i < half; ++i) {
            const double inv_freq = pow(theta, -2.0 * (double)i / (double)D);
            const double a = (double)p * inv_freq;
            cos_t[p * half + i] = (float)cos(a);
            sin_t[p * half + i] = (float)sin(a);
        }
    }
    return 0;
}

/* y[m][h][:] = RoPE(x[m][h][:], pos[m]); x rows are x_stride elements apart
 * and hold `heads` head vectors of D back to back; y is [M][heads][D]. */
int or_rope(const uint16_t *x, uint16_t *y, const int32_t *pos, int64_t M, int heads,
            int D, int64_t x_stride, const float *cos_t, const float *sin_t,
            int64_t max_pos)
{
    if (M < 0 || heads <= 0 || D <= 0 || D % 2 != 0 || x_stride < (int64_t)heads * D)
        return -1;
    const int half = D / 2;
    for (int64_t m = 0; m < M; ++m) {
        const int64_t p = pos[m];
        if (p < 0 || p >= max_pos)
            return -1;
        const float *c = cos_t + p * half;
        const float *s = sin_t + p * half;
        for (int h = 0; h < heads; ++h) {
            const uint16_t *xr = x + m * x_stride + (int64_t)h * D;
            uint16_t *yr = y + (m * heads + h) * (int64_t)D;
            for (int i = 0; i < half; ++i) {
                const float a = lay_bf16_to_f32(xr[i]);
                const float b = lay_bf16_to_f32(xr[i + half]);
                const float ac = a * c[i], bs = b * s[i];
                const float bc = b * c[i], as = a * s[i];
                yr[i] = or_f32_to_bf16(ac - bs);
                yr[i + half] = or_f32_to_bf16(bc + as);
            }
        }
    }
    return 0;
}

/* y[m][f] = bf16(silu(gu[m][f]) * gu[m][F + f]), gu is [M][2F]. */
int or_silu_mul(const uint16_t *gu, uint16_t *y, int64_t M, int64_t F)
{
    if (M < 0 || F <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t f = 0; f < F; ++f) {
            const float g = lay_bf16_to_f32(gu[m * 2 * F + f]);
            const float u = lay_bf16_to_f32(gu[m * 2 * F + F + f]);
            const float e = expf(-g);
            const float den = 1.0f + e;
            const float sg = g / den;
            y[m * F + f] = or_f32_to_bf16(sg * u);
        }
    }
    return 0;
}

/* y = bf16(a + b), element-wise over n values. */
int or_add(const uint16_t *a, const uint16_t *b, uint16_t *y, int64_t n)
{
    if (n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        y[i] = or_f32_to_bf16(lay_bf16_to_f32(a[i]) + lay_bf16_to_f32(b[i]));
    return 0;
}
