/*
 * bi_oracle.c -- plain, slow CPU oracle for the batch-invariant forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant generator
 * with the HIP kernels: every schedule constant below is restated here from
 * the written schedule, not included from the product.
 *
 * Sources (web pages; cited by title and section):
 *   [Article]  "LLM inference determinism engineering in depth: from float
 *              non-associativity and batch invariance to reproducible kernels"
 *              (ybb.press, ai-applications/14528).
 *   [LLM-42]   "LLM-42: Enabling Determinism in LLM Inference with Verified
 *              Speculation (SOSP 2026)" -- ai-infra-wiki digest.
 *   [Vosti]    arxivdaily 2609.38981, abstract of the Vosti engine.
 *
 * Two kinds of function:
 *   or_*        The fixed reduction schedule, in fp32 from bf16 inputs, exactly
 *               as written in the schedule: per-element fp32 operations in the
 *               order the schedule fixes.  Loops run across independent outputs
 *               (columns n, channels h, dims d) only; no single sum is split,
 *               blocked or reordered beyond what the schedule states.
 *   or_*_exact  The plain mathematical definition in fp64, used to pin the
 *               schedule oracle (error bounds, special cases).
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared.
 * FP contraction is off, so every a*b+c below is two roundings unless fmaf()
 * is written out.  x86-64 SSE arithmetic evaluates float in float
 * (FLT_EVAL_METHOD == 0), so each float operation is one IEEE rounding.
 *
 * Parity status of each function is stated in its comment.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "bi_oracle.h"

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                              */
/* ------------------------------------------------------------------------ */

/* bf16 is the top half of an IEEE binary32: widening is exact. */
static float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Narrowing with round-to-nearest, ties-to-even, done on the bit pattern.
 * NaN stays NaN (quiet bit set).  [Article] section 5 warns against any
 * reduced-precision intermediate; the only narrowing on the path is this
 * final store. */
uint16_t or_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float or_bf16_value(uint16_t b) { return or_bf16_to_f32(b); }

/* ------------------------------------------------------------------------ */
/* fp32 left fold -- the primitive behind every ordered sum below.            */
/* [Article] section 2.1: IEEE addition is not associative, so the grouping   */
/* is part of the result.  A left fold is ((v0 + v1) + v2) + ...              */
/* ------------------------------------------------------------------------ */
float or_fold_f32(const float *v, int64_t n)
{
    if (n <= 0)
        return 0.0f;
    float s = v[0];
    for (int64_t i = 1; i < n; ++i)
        s = s + v[i];
    return s;
}

/* ------------------------------------------------------------------------ */
/* GEMM: y[M,N] = bf16( x[M,K] . W[K,N] )                                     */
/* ------------------------------------------------------------------------ */
/*
 * Schedule (fixed; depends on K only, never on M):
 *   KB = 32   one K-block = the contraction depth of one bf16 matrix-core op.
 *   KC = 512  one segment = 16 K-blocks, accumulated from +0.
 *   S  = ceil(K / KC) segments, folded left in index order 0..S-1.
 * [Article] section 4: fixed tiling, no float atomics, and a K split written
 * as per-slice partials into a fixed workspace that a second stage adds in the
 * fixed index order 0..SPLIT-1 (read here as a serial left fold).
 * [Article] section 2.2: the split-k atomicAdd tail is the pattern replaced.
 *
 * Within one K-block the 32 bf16 products are exact in fp32 (8-bit by 8-bit
 * significands); they are summed left to right from +0, and the block sum is
 * added to the segment accumulator with one rounding.  How the matrix core
 * associates the 32 products inside one instruction is not documented, so
 * this in-block order is a model: parity at that level is unpinned and is
 * covered by the output tolerance.  Every order above the block (block order,
 * segment start from +0, segment fold order) is pinned by exact tests.
 *
 * Loops run over rows m and, innermost, over independent columns n; each
 * output element sees exactly the sequence of roundings written above.
 *
 * x row-major [M,K], W row-major [K,N] (the weight multiplies from the right,
 * as in the article's section-1 demo), y row-major [M,N].  y32 (optional,
 * may be NULL) receives the fp32 value before narrowing.
 */
#define OR_GEMM_KB 32
#define OR_GEMM_KC 512

int or_gemm(const uint16_t *x, const uint16_t *w, uint16_t *y, float *y32,
            int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0)
        return -1;
    float *total = (float *)malloc((size_t)N * sizeof(float));
    float *seg = (float *)malloc((size_t)N * sizeof(float));
    float *blk = (float *)malloc((size_t)N * sizeof(float));
    float *wrow = (float *)malloc((size_t)N * sizeof(float));
    if (!total || !seg || !blk || !wrow) {
        free(total); free(seg); free(blk); free(wrow);
        return -2;
    }
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xm = x + m * K;
        for (int64_t s0 = 0; s0 < K; s0 += OR_GEMM_KC) {
            int64_t s1 = s0 + OR_GEMM_KC < K ? s0 + OR_GEMM_KC : K;
            for (int64_t n = 0; n < N; ++n)
                seg[n] = 0.0f;
            for (int64_t b0 = s0; b0 < s1; b0 += OR_GEMM_KB) {
                int64_t b1 = b0 + OR_GEMM_KB < s1 ? b0 + OR_GEMM_KB : s1;
                for (int64_t n = 0; n < N; ++n)
                    blk[n] = 0.0f;
                for (int64_t k = b0; k < b1; ++k) {
                    float xv = or_bf16_to_f32(xm[k]);
                    const uint16_t *wk = w + k * N;
                    for (int64_t n = 0; n < N; ++n)
                        wrow[n] = or_bf16_to_f32(wk[n]);
                    for (int64_t n = 0; n < N; ++n)
                        blk[n] = blk[n] + xv * wrow[n]; /* product exact */
                }
                for (int64_t n = 0; n < N; ++n)
                    seg[n] = seg[n] + blk[n];
            }
            if (s0 == 0) {
                for (int64_t n = 0; n < N; ++n)
                    total[n] = seg[n];
            } else {
                for (int64_t n = 0; n < N; ++n)
                    total[n] = total[n] + seg[n];
            }
        }
        for (int64_t n = 0; n < N; ++n) {
            y[m * N + n] = or_f32_to_bf16(total[n]);
            if (y32)
                y32[m * N + n] = total[n];
        }
    }
    free(total); free(seg); free(blk); free(wrow);
    return 0;
}

/* The definition: y = x.W summed in fp64.  Each bf16 product is exact in fp64
 * and the fp64 sum's error (<= K * 2^-53 * sum|x w|) is far below a bf16 ulp,
 * so this stands in for the exact value. */
int or_gemm_exact(const uint16_t *x, const uint16_t *w, double *y,
                  int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xv = (double)or_bf16_to_f32(x[m * K + k]);
            for (int64_t n = 0; n < N; ++n)
                y[m * N + n] += xv * (double)or_bf16_to_f32(w[k * N + n]);
        }
    }
    return 0;
}

/* Per-element sum of |x||w|, the scale of the rounding-error bound. */
int or_gemm_absdot(const uint16_t *x, const uint16_t *w, double *a,
                   int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N <= 0 || K <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n)
            a[m * N + n] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xv = fabs((double)or_bf16_to_f32(x[m * K + k]));
            for (int64_t n = 0; n < N; ++n)
                a[m * N + n] += xv * fabs((double)or_bf16_to_f32(w[k * N + n]));
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm: y[m,h] = bf16( (x[m,h] * r_m) * g[h] ),                           */
/*          r_m = 1 / sqrt( sum_h x[m,h]^2 / H + eps )                         */
/* ------------------------------------------------------------------------ */
/*
 * The pages name normalization only as one of the reductions whose schedule a
 * dynamic batch changes ([LLM-42] problem statement; [Article] section 2.2).
 * The formula is the Llama RMSNorm with eps inside the square root; g is bf16;
 * there is no intermediate narrowing; the order is (x*r)*g.
 *
 * Schedule (fixed; depends on H only): one row is reduced by 256 lanes in
 * four groups of 64.
 *   lane t, t = 0..255, sums x^2 left to right over the channels
 *       h = 8*(t + 256*i) + j,  i = 0, 1, ... while h < H,  j = 0..7
 *   (x^2 of a bf16 value is exact in fp32);
 *   within each group of 64 lanes: for o = 32, 16, 8, 4, 2, 1 every lane l
 *       replaces its value v_l by v_l + v_(l xor o)  (all lanes end equal);
 *   the four group results are folded ((w0 + w1) + w2) + w3;
 *   ms = ss / H; d = ms + eps; r = 1 / sqrt(d), each correctly rounded.
 * Parity: every operation is an IEEE basic operation, so the kernel can match
 * this bit for bit.  Pinned by fp64 brute force and closed-form rows.
 */
#define OR_RMS_LANES 256
#define OR_RMS_GROUP 64
#define OR_RMS_VEC 8

static float or_rms_rowsum(const uint16_t *xr, int64_t H)
{
    float part[OR_RMS_LANES];
    for (int t = 0; t < OR_RMS_LANES; ++t) {
        float a = 0.0f;
        for (int64_t i = 0;; ++i) {
            int64_t base = (int64_t)OR_RMS_VEC * (t + (int64_t)OR_RMS_LANES * i);
            if (base >= H)
                break;
            for (int j = 0; j < OR_RMS_VEC; ++j) {
                int64_t h = base + j;
                if (h < H) {
                    float v = or_bf16_to_f32(xr[h]);
                    a = a + v * v;
                }
            }
        }
        part[t] = a;
    }
    float gsum[OR_RMS_LANES / OR_RMS_GROUP];
    for (int g = 0; g < OR_RMS_LANES / OR_RMS_GROUP; ++g) {
        float v[OR_RMS_GROUP], nv[OR_RMS_GROUP];
        for (int l = 0; l < OR_RMS_GROUP; ++l)
            v[l] = part[g * OR_RMS_GROUP + l];
        for (int o = OR_RMS_GROUP / 2; o >= 1; o /= 2) {
            for (int l = 0; l < OR_RMS_GROUP; ++l)
                nv[l] = v[l] + v[l ^ o];
            memcpy(v, nv, sizeof v);
        }
        gsum[g] = v[0];
    }
    return or_fold_f32(gsum, OR_RMS_LANES / OR_RMS_GROUP);
}

int or_rmsnorm(const uint16_t *x, const uint16_t *g, uint16_t *y, float *rinv,
               int64_t M, int64_t H, float eps)
{
    if (M < 0 || H <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t *xr = x + m * H;
        float ss = or_rms_rowsum(xr, H);
        float ms = ss / (float)H;
        float d = ms + eps;
        float r = 1.0f / sqrtf(d);
        if (rinv)
            rinv[m] = r;
        for (int64_t h = 0; h < H; ++h) {
            float t = or_bf16_to_f32(xr[h]) * r;
            y[m * H + h] = or_f32_to_bf16(t * or_bf16_to_f32(g[h]));
        }
    }
    return 0;
}

int or_rmsnorm_exact(const uint16_t *x, const uint16_t *g, double *y,
                     int64_t M, int64_t H, double eps)
{
    if (M < 0 || H <= 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double v = (double)or_bf16_to_f32(x[m * H + h]);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / (double)H + eps);
        for (int64_t h = 0; h < H; ++h)
            y[m * H + h] = (double)or_bf16_to_f32(x[m * H + h]) * r *
                           (double)or_bf16_to_f32(g[h]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Paged decode attention                                                     */
/* ------------------------------------------------------------------------ */
/*
 * For request b and query head h (kv head hk = h / (Hq/Hkv)):
 *   out[b,h,:] = softmax_t( scale * q[b,h,:].k_t ) . v_t   over t < L_b,
 * where token t's key and value live in page block_table[b][t / PS], slot
 * t % PS.  The pages give the operation only as "attention" with a paged,
 * prefix-shared KV cache whose layout must not change the bits ([Vosti]
 * abstract; [LLM-42] problem statement).  Readings: scale = 1/sqrt(D), no
 * mask besides t < L_b, GQA group = Hq/Hkv consecutive heads, ctx_len <= 0
 * gives zeros.
 *
 * kv_pages layout: [page][K|V][kv_head][slot][d], so one (page, K|V, head)
 * block is PS*D contiguous bf16.
 *
 * Schedule (fixed; depends on D, PS, Hq, Hkv only, never on the batch, the
 * page placement or the longest context):
 *   chunks of C = 256 tokens, c = 0 .. ceil(L/C)-1, each starting from
 *   m = -inf, l = 0, acc = 0; inside a chunk, tiles of T = 64 tokens in order:
 *     s_t   = (sum_d q_d k_td, left to right from +0, products exact) * scale
 *     m'    = max(m, max_t s_t)
 *     alpha = exp(m - m')            (alpha = 0 while m = -inf)
 *     l     = l * alpha, then l = l + p_t for t in order, p_t = exp(s_t - m')
 *     acc_d = acc_d * alpha, then acc_d = fma(p_t, v_td, acc_d) for t in order
 *     m     = m'
 *   combine in chunk order ([Article] section 4, ordered second stage):
 *     M* = max_c m_c, w_c = exp(m_c - M*),
 *     Lsum = fma(l_c, w_c, Lsum) and O_d = fma(acc_c,d, w_c, O_d), c = 0..,
 *     out_d = bf16(O_d / Lsum).
 * Parity: the exponential (host expf vs the device's own exp) and the
 * grouping inside the q.k dot (the device sums 32-dimension blocks on the
 * matrix cores, the blocks in order) are unpinned at the last-bit level and
 * covered by the tolerance; everything else follows the same steps.  Pinned by fp64
 * brute force, the one-token case (out = v_0 exactly), constant V, q = 0,
 * and page-layout invariance.
 */
#define OR_ATT_C 256
#define OR_ATT_T 64

static const uint16_t *or_kv_row(const uint16_t *kv, const int32_t *bt_row,
                                 int64_t t, int which, int hk, int Hkv, int PS,
                                 int D)
{
    int64_t page = bt_row[t / PS];
    int64_t slot = t % PS;
    return kv + (((page * 2 + which) * Hkv + hk) * PS + slot) * D;
}

int or_paged_decode_attn(const uint16_t *q, const uint16_t *kv,
                         const int32_t *block_table, const int32_t *ctx_lens,
                         uint16_t *out, int64_t B, int Hq, int Hkv, int D,
                         int PS, int64_t max_blocks, float scale)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || PS <= 0)
        return -1;
    const int G = Hq / Hkv;
    float *acc = (float *)malloc((size_t)D * sizeof(float));
    float *O = (float *)malloc((size_t)D * sizeof(float));
    float *qf = (float *)malloc((size_t)D * sizeof(float));
    float s[OR_ATT_T], p[OR_ATT_T];
    if (!acc || !O || !qf) {
        free(acc); free(O); free(qf);
        return -2;
    }
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = ctx_lens[b];
        const int32_t *btr = block_table + b * max_blocks;
        for (int h = 0; h < Hq; ++h) {
            uint16_t *o = out + (b * Hq + h) * D;
            if (L <= 0) {
                for (int d = 0; d < D; ++d)
                    o[d] = 0;
                continue;
            }
            const int hk = h / G;
            for (int d = 0; d < D; ++d)
                qf[d] = or_bf16_to_f32(q[(b * Hq + h) * D + d]);
            const int64_t nc = (L + OR_ATT_C - 1) / OR_ATT_C;
            float *cm = (float *)malloc((size_t)nc * sizeof(float));
            float *cl = (float *)malloc((size_t)nc * sizeof(float));
            float *cacc = (float *)malloc((size_t)nc * D * sizeof(float));
            if (!cm || !cl || !cacc) {
                free(cm); free(cl); free(cacc);
                free(acc); free(O); free(qf);
                return -2;
            }
            for (int64_t c = 0; c < nc; ++c) {
                const int64_t cend = (c + 1) * OR_ATT_C < L ? (c + 1) * OR_ATT_C : L;
                float m = -INFINITY, l = 0.0f;
                for (int d = 0; d < D; ++d)
                    acc[d] = 0.0f;
                for (int64_t t0 = c * OR_ATT_C; t0 < cend; t0 += OR_ATT_T) {
                    const int64_t t1 = t0 + OR_ATT_T < cend ? t0 + OR_ATT_T : cend;
                    const int nt = (int)(t1 - t0);
                    float mt = -INFINITY;
                    for (int i = 0; i < nt; ++i) {
                        const uint16_t *kr = or_kv_row(kv, btr, t0 + i, 0, hk, Hkv, PS, D);
                        float dot = 0.0f;
                        for (int d = 0; d < D; ++d)
                            dot = dot + qf[d] * or_bf16_to_f32(kr[d]);
                        s[i] = dot * scale;
                        if (s[i] > mt)
                            mt = s[i];
                    }
                    const float mn = m > mt ? m : mt;
                    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - mn);
                    for (int i = 0; i < nt; ++i)
                        p[i] = expf(s[i] - mn);
                    l = l * alpha;
                    for (int i = 0; i < nt; ++i)
                        l = l + p[i];
                    for (int d = 0; d < D; ++d)
                        acc[d] = acc[d] * alpha;
                    for (int i = 0; i < nt; ++i) {
                        const uint16_t *vr = or_kv_row(kv, btr, t0 + i, 1, hk, Hkv, PS, D);
                        for (int d = 0; d < D; ++d)
                            acc[d] = fmaf(p[i], or_bf16_to_f32(vr[d]), acc[d]);
                    }
                    m = mn;
                }
                cm[c] = m;
                cl[c] = l;
                memcpy(cacc + c * D, acc, (size_t)D * sizeof(float));
            }
            float Mx = -INFINITY;
            for (int64_t c = 0; c < nc; ++c)
                if (cm[c] > Mx)
                    Mx = cm[c];
            float Ls = 0.0f;
            for (int d = 0; d < D; ++d)
                O[d] = 0.0f;
            for (int64_t c = 0; c < nc; ++c) {
                const float wgt = expf(cm[c] - Mx);
                Ls = fmaf(cl[c], wgt, Ls);
                for (int d = 0; d < D; ++d)
                    O[d] = fmaf(cacc[c * D + d], wgt, O[d]);
            }
            for (int d = 0; d < D; ++d)
                o[d] = or_f32_to_bf16(O[d] / Ls);
            free(cm); free(cl); free(cacc);
        }
    }
    free(acc); free(O); free(qf);
    return 0;
}

/* The definition in fp64: a single softmax over all L tokens (no chunks, no
 * online rescaling), max-subtracted for range only. */
int or_paged_decode_attn_exact(const uint16_t *q, const uint16_t *kv,
                               const int32_t *block_table,
                               const int32_t *ctx_lens, double *out, int64_t B,
                               int Hq, int Hkv, int D, int PS,
                               int64_t max_blocks, double scale)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || PS <= 0)
        return -1;
    const int G = Hq / Hkv;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t L = ctx_lens[b];
        const int32_t *btr = block_table + b * max_blocks;
        for (int h = 0; h < Hq; ++h) {
            double *o = out + (b * Hq + h) * D;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            if (L <= 0)
                continue;
            const int hk = h / G;
            double *s = (double *)malloc((size_t)L * sizeof(double));
            if (!s)
                return -2;
            double mx = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                const uint16_t *kr = or_kv_row(kv, btr, t, 0, hk, Hkv, PS, D);
                double dot = 0.0;
                for (int d = 0; d < D; ++d)
                    dot += (double)or_bf16_to_f32(q[(b * Hq + h) * D + d]) *
                           (double)or_bf16_to_f32(kr[d]);
                s[t] = dot * scale;
                if (s[t] > mx)
                    mx = s[t];
            }
            double den = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                s[t] = exp(s[t] - mx);
                den += s[t];
            }
            for (int64_t t = 0; t < L; ++t) {
                const uint16_t *vr = or_kv_row(kv, btr, t, 1, hk, Hkv, PS, D);
                for (int d = 0; d < D; ++d)
                    o[d] += s[t] * (double)or_bf16_to_f32(vr[d]);
            }
            for (int d = 0; d < D; ++d)
                o[d] /= den;
            free(s);
        }
    }
    return 0;
}
