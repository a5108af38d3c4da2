// bi_sample.hip -- per-request sampling and the commit-or-rollback step of
// grouped verification.
//
// Sampling (Determinism article, section 6, item 3: a counter-based
// generator of the Philox family keyed by request and step, never a shared
// stream).  Row m's token depends only on its logits row, its request seed
// and its step:
//   generator  Philox4x64-10 (Salmon et al., SC 2011), key (seed, 0),
//              counter (v / 4, step, 0, 0); entry v takes word v % 4;
//   uniform    u = ((word >> 41) + 1/2) * 2^-23, exact in fp32, in (0, 1);
//   T > 0      Gumbel-max: score = l / T + (-log(-log u)), fp32;
//   T <= 0     greedy: score = l;
//   token      the first index of the largest score (NaN counts as -inf).
// The maximum with first-index ties is exact and order-free, so neither the
// split of the vocabulary over workgroups nor any reduction tree can change
// the token.
//
// Commit or rollback (LLM-42 digest, method: a verified prefix is committed;
// at the first mismatch the later candidates are discarded and decoding
// resumes from the committed prefix).
#include <math.h>

#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                              uint64_t k0, uint64_t k1, uint64_t (&out)[4]) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t a = 0xD2E7470EE14C6C93ULL * c0;
    const uint64_t ah = __umul64hi(0xD2E7470EE14C6C93ULL, c0);
    const uint64_t b = 0xCA5A826395121157ULL * c2;
    const uint64_t bh = __umul64hi(0xCA5A826395121157ULL, c2);
    c0 = bh ^ c1 ^ k0;
    c1 = b;
    c2 = ah ^ c3 ^ k1;
    c3 = a;
    k0 += 0x9E3779B97F4A7C15ULL;
    k1 += 0xBB67AE8584CAA73BULL;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// (score, index) order: larger score first, then smaller index
__device__ __forceinline__ bool sample_better(float s, int i, float bs, int bi) {
  return s > bs || (s == bs && i < bi);
}

// Two launches.  sample_chunk_kernel: grid = (SMP_CHUNKS, M), block = 256;
// workgroup p takes the vocabulary entries of chunk p (whole 4-entry Philox
// blocks), lane t its blocks t, t + 256, ..., and writes the chunk's best
// (score, index) to the workspace.  sample_pick_kernel: one 64-lane wave
// per row takes the best of the chunks.  The maximum with first-index ties
// is exact and does not depend on how the entries are grouped.
static constexpr int SMP_CHUNKS = 32;

__global__ __launch_bounds__(256) void sample_chunk_kernel(
    const uint16_t* __restrict__ logits, int64_t V, const uint64_t* __restrict__ seeds,
    const uint64_t* __restrict__ steps, const float* __restrict__ temps,
    float* __restrict__ best_s, int32_t* __restrict__ best_i) {
  __shared__ float rs[4];
  __shared__ int ri[4];
  const int p = blockIdx.x;
  const int64_t m = blockIdx.y;
  const int64_t nblk = (V + 3) / 4;
  const int64_t per = (nblk + SMP_CHUNKS - 1) / SMP_CHUNKS;  // Philox blocks per chunk
  const int64_t b0 = p * per, b1 = min(nblk, b0 + per);
  const uint16_t* row = logits + m * V;
  const float T = temps[m];
  const bool greedy = !(T > 0.0f);
  const uint64_t seed = seeds[m], step = steps[m];
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int64_t b = b0 + threadIdx.x; b < b1; b += 256) {
    uint64_t r[4] = {0, 0, 0, 0};
    if (!greedy) philox4x64_10((uint64_t)b, step, 0, 0, seed, 0, r);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t v = b * 4 + w;
      if (v < V) {
        const float l = __uint_as_float((uint32_t)row[v] << 16);
        float s;
        if (greedy) {
          s = l;
        } else {
          const float u = ((float)(r[w] >> 41) + 0.5f) * 0x1p-23f;
          const float y = logf(u);
          const float z = logf(-y);
          const float q = l / T;  // IEEE division
          s = q + (-z);
        }
        if (s != s) s = -INFINITY;
        if (sample_better(s, (int)v, best, bidx)) {
          best = s;
          bidx = (int)v;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float os = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bidx, o, 64);
    if (sample_better(os, oi, best, bidx)) {
      best = os;
      bidx = oi;
    }
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    rs[wave] = best;
    ri[wave] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (sample_better(rs[w], ri[w], best, bidx)) {
        best = rs[w];
        bidx = ri[w];
      }
    best_s[m * SMP_CHUNKS + p] = best;
    best_i[m * SMP_CHUNKS + p] = bidx;
  }
}

__global__ __launch_bounds__(64) void sample_pick_kernel(const float* __restrict__ best_s,
                                                         const int32_t* __restrict__ best_i,
                                                         int32_t* __restrict__ tokens) {
  const int64_t m = blockIdx.x;
  const int l = threadIdx.x;
  float best = l < SMP_CHUNKS ? best_s[m * SMP_CHUNKS + l] : -INFINITY;
  int bidx = l < SMP_CHUNKS ? best_i[m * SMP_CHUNKS + l] : 0x7fffffff;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float os = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bidx, o, 64);
    if (sample_better(os, oi, best, bidx)) {
      best = os;
      bidx = oi;
    }
  }
  if (l == 0) tokens[m] = bidx;
}

// One lane per request: the window's leading matches are accepted; at the
// first mismatch the recompute's token is committed and the rest dropped.
__global__ __launch_bounds__(256) void verify_commit_kernel(
    const int32_t* __restrict__ cand, const int32_t* __restrict__ ver,
    const int32_t* __restrict__ row_start, int R, int rows, int32_t* __restrict__ accepted,
    int32_t* __restrict__ commit_len, int32_t* __restrict__ fix_token) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  // window rows clamped to [0, rows), whatever row_start holds
  const int s = min(max(0, (int)row_start[r]), rows);
  const int w = min(max(s, (int)row_start[r + 1]), rows) - s;
  int a = 0;
  while (a < w && cand[s + a] == ver[s + a]) ++a;
  accepted[r] = a;
  commit_len[r] = commit_len[r] + (a < w ? a + 1 : w);
  fix_token[r] = a < w ? ver[s + a] : -1;
}

size_t sample_ws_bytes(int64_t M) { return (size_t)M * SMP_CHUNKS * 8; }

int launch_sample(const uint16_t* logits, int64_t M, int64_t V, const uint64_t* seeds,
                  const uint64_t* steps, const float* temps, int32_t* tokens, void* ws,
                  hipStream_t stream) {
  float* bs = (float*)ws;
  int32_t* bidx = (int32_t*)(bs + M * SMP_CHUNKS);
  hipLaunchKernelGGL(sample_chunk_kernel, dim3(SMP_CHUNKS, (unsigned)M), dim3(256), 0, stream,
                     logits, V, seeds, steps, temps, bs, bidx);
  if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
  hipLaunchKernelGGL(sample_pick_kernel, dim3((unsigned)M), dim3(64), 0, stream, bs, bidx,
                     tokens);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

int launch_verify_commit(const int32_t* cand, const int32_t* ver, const int32_t* row_start, int R,
                         int rows, int32_t* accepted, int32_t* commit_len, int32_t* fix_token,
                         hipStream_t stream) {
  hipLaunchKernelGGL(verify_commit_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0,
                     stream, cand, ver, row_start, R, rows, accepted, commit_len, fix_token);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
