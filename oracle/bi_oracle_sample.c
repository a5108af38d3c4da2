/*
 * bi_oracle_sample.c -- plain CPU oracle for per-request sampling.
 *
 * TEST INFRASTRUCTURE ONLY, like bi_oracle.c: nothing in the product library
 * links, loads or calls this file, and it shares no code with the HIP path.
 *
 * Source: the Determinism article, section 6 (serving-side controls), item
 * 3: draw each request's random numbers from a counter-based generator of
 * the Philox family keyed by the request and the decoding step, instead of a
 * shared stream, so that a token never depends on what else was sampled.
 * The pages name the generator family and the (request, step) keying only;
 * the rest is this reading:
 *
 *   generator: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
 *     random numbers: as easy as 1, 2, 3", SC 2011): ten rounds on a
 *     4 x 64-bit counter with a 2 x 64-bit key; each round multiplies words
 *     0 and 2 by fixed odd constants into 128-bit products, and the new
 *     counter is (hi(c2 m1) ^ c1 ^ k0, lo(c2 m1), hi(c0 m0) ^ c3 ^ k1,
 *     lo(c0 m0)); the key is bumped by the two Weyl constants between
 *     rounds.
 *   keying: key = (seed of the request, 0), counter = (v / 4, step, 0, 0);
 *     vocabulary entry v takes 64-bit word v % 4 of that block.
 *   uniform: u = ((word >> 41) + 1/2) * 2^-23: a 24-bit odd numerator over
 *     2^24, exact in fp32, in (0, 1) (never 0, never 1).
 *   temperature T > 0: Gumbel-max sampling, score_v = l_v / T + g_v with
 *     g_v = -log(-log(u_v)), all fp32 (one IEEE division, two logf, one
 *     negation, one addition); the token is the first index of the largest
 *     score (NaN scores count as -infinity).
 *   T <= 0 (or NaN): greedy, score_v = l_v.
 *
 * Parity: Philox is bit-exact (integer); with T > 0 the logarithms are the
 * platform's, so a token is unique unless two scores lie within a few ulp.
 */
#include <math.h>
#include <stdint.h>

#include "bi_oracle.h"

typedef unsigned __int128 or_u128;

void or_philox4x64(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
  const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
  uint64_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint64_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    const or_u128 p0 = (or_u128)M0 * c[0];
    const or_u128 p1 = (or_u128)M1 * c[2];
    const uint64_t n0 = (uint64_t)(p1 >> 64) ^ c[1] ^ k0;
    const uint64_t n1 = (uint64_t)p1;
    const uint64_t n2 = (uint64_t)(p0 >> 64) ^ c[3] ^ k1;
    const uint64_t n3 = (uint64_t)p0;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
    k0 += W0;
    k1 += W1;
  }
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

static float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return v.f;
}

float or_sample_uniform(uint64_t seed, uint64_t step, int64_t v) {
  const uint64_t ctr[4] = {(uint64_t)(v / 4), step, 0, 0};
  const uint64_t key[2] = {seed, 0};
  uint64_t r[4];
  or_philox4x64(ctr, key, r);
  return ((float)(r[v % 4] >> 41) + 0.5f) * 0x1p-23f;
}

int or_sample(const uint16_t *logits, int64_t M, int64_t V, const uint64_t *seeds,
              const uint64_t *steps, const float *temps, int32_t *tokens, float *best_score,
              float *second_score) {
  if (!logits || !seeds || !steps || !temps || !tokens || M < 0 || V <= 0) return -1;
  for (int64_t m = 0; m < M; ++m) {
    const float T = temps[m];
    const int greedy = !(T > 0.0f);
    float best = -INFINITY, second = -INFINITY;
    int64_t bidx = -1;
    for (int64_t v = 0; v < V; ++v) {
      const float l = bf16_to_f32(logits[m * V + v]);
      float s;
      if (greedy) {
        s = l;
      } else {
        const float u = or_sample_uniform(seeds[m], steps[m], v);
        const float y = logf(u);        /* < 0 */
        const float z = logf(-y);
        const float q = l / T;
        s = q + (-z);
      }
      if (s != s) s = -INFINITY;
      if (bidx < 0 || s > best) {
        if (bidx >= 0) second = best;
        best = s;
        bidx = v;
      } else if (s > second) {
        second = s;
      }
    }
    tokens[m] = (int32_t)bidx;
    if (best_score) best_score[m] = best;
    if (second_score) second_score[m] = second;
  }
  return 0;
}
