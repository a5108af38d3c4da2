// bi_layer.hip -- the element-wise steps that join the batch-invariant
// kernels into a Llama-style decoder layer: token embedding, rotary position
// embedding, KV-cache append, SiLU-gated product and residual add.
//
// Every output element depends on its own row's inputs only, with a fixed
// sequence of fp32 operations and one bf16 rounding (round to nearest even),
// so none of these can move with the batch (the LLM-42 digest's problem
// statement: a token's logits must not depend on what it is verified with).
// Formulas (the pages name the steps, not their arithmetic; standard Llama):
//   RoPE, rotate-half pairs (i, i + D/2):
//     y_i       = bf16(x_i c_i(p) - x_{i+D/2} s_i(p))
//     y_{i+D/2} = bf16(x_{i+D/2} c_i(p) + x_i s_i(p))
//     each product rounded to fp32 before the sum (no fused multiply-add);
//     c, s from a table built on the host: angle p * theta^(-2i/D) in double,
//     cos and sin each rounded once to fp32.
//   SiLU product of [gate | up]: y = bf16((g / (1 + exp(-g))) * u), fp32.
//   Residual add: y = bf16(a + b), one fp32 addition.
#include <math.h>

#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

// ---------------------------------------------------------------------------
// Embedding: out[m, :] = table[tokens[m], :]; ids outside [0, V) give zeros.
// grid = M, block = 256; 16-byte chunks.
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens,
                                                    const uint16_t* __restrict__ table,
                                                    uint16_t* __restrict__ out, int64_t V,
                                                    int64_t H) {
  const int64_t m = blockIdx.x;
  const int64_t tok = tokens[m];
  const bool ok = tok >= 0 && tok < V;
  const u32x4_t* src = (const u32x4_t*)(table + (ok ? tok : 0) * H);
  u32x4_t* dst = (u32x4_t*)(out + m * H);
  for (int64_t c = threadIdx.x; c < H / 8; c += 256)
    dst[c] = ok ? src[c] : u32x4_t{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// RoPE of `heads` head vectors of D = 128 per row.  block = 256 lanes, 16
// per head vector (16 heads per workgroup): lane i of a head owns the pairs
// (4i .. 4i+3, 4i+64 .. 4i+67), read and written 8 bytes at a time.
// grid = (M, ceil(heads / 16)).  x rows are x_stride elements apart; out is
// [M, heads, D].  Positions outside [0, max_pos) give zeros.
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* __restrict__ x,
                                                   int64_t x_stride, uint16_t* __restrict__ out,
                                                   const int32_t* __restrict__ pos,
                                                   const float* __restrict__ cos_t,
                                                   const float* __restrict__ sin_t, int heads,
                                                   int64_t max_pos) {
  constexpr int D = 128, HALF = 64;
  const int64_t m = blockIdx.x;
  const int h = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int i = (threadIdx.x & 15) * 4;
  if (h >= heads) return;
  const int64_t p = pos[m];
  uint16_t* o = out + (m * heads + h) * D;
  if (p < 0 || p >= max_pos) {
    *(u32x2_t*)(o + i) = u32x2_t{0u, 0u};
    *(u32x2_t*)(o + i + HALF) = u32x2_t{0u, 0u};
    return;
  }
  const uint16_t* xr = x + m * x_stride + (int64_t)h * D;
  const u32x2_t lo = *(const u32x2_t*)(xr + i);         // x_i .. x_{i+3}
  const u32x2_t hi = *(const u32x2_t*)(xr + i + HALF);  // x_{i+64} .. x_{i+67}
  const f32x4_t c = *(const f32x4_t*)(cos_t + p * HALF + i);
  const f32x4_t s = *(const f32x4_t*)(sin_t + p * HALF + i);
  const float a[4] = {bf16_lo(lo.x), bf16_hi(lo.x), bf16_lo(lo.y), bf16_hi(lo.y)};
  const float b[4] = {bf16_lo(hi.x), bf16_hi(hi.x), bf16_lo(hi.y), bf16_hi(hi.y)};
  float r0[4], r1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float ac = a[j] * c[j], bs = b[j] * s[j];  // rounded products (no contraction)
    const float bc = b[j] * c[j], as = a[j] * s[j];
    r0[j] = ac - bs;
    r1[j] = bc + as;
  }
  *(u32x2_t*)(o + i) = u32x2_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3])};
  *(u32x2_t*)(o + i + HALF) = u32x2_t{pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
}

// ---------------------------------------------------------------------------
// KV append: row m's key and value head vectors go to slot pos[m] % PS of
// page block_table[m][pos[m] / PS] of the [P][2][Hkv][PS][D] cache.  grid =
// (M, Hkv), block = 32: lanes 0..15 copy K, 16..31 copy V, 16 bytes each.
// Rows whose page is missing or out of range are skipped.
__global__ __launch_bounds__(32) void kv_append_kernel(
    const uint16_t* __restrict__ k, int64_t k_stride, const uint16_t* __restrict__ v,
    int64_t v_stride, uint16_t* __restrict__ kv, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ pos, int Hkv, int max_blocks, int64_t num_pages) {
  constexpr int D = 128, PS = 16;
  const int64_t m = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t p = pos[m];
  if (p < 0 || p / PS >= max_blocks) return;
  const int64_t page = block_table[m * max_blocks + p / PS];
  if (page < 0 || page >= num_pages) return;
  const int which = lane >> 4;  // 0: K, 1: V
  const int c = lane & 15;
  const uint16_t* src = which == 0 ? k + m * k_stride + (int64_t)h * D
                                   : v + m * v_stride + (int64_t)h * D;
  uint16_t* dst = kv + (((page * 2 + which) * Hkv + h) * PS + p % PS) * D;
  ((u32x4_t*)dst)[c] = ((const u32x4_t*)src)[c];
}

// ---------------------------------------------------------------------------
// SiLU product: out[m, f] = bf16(silu(gu[m, f]) * gu[m, F + f]).
// grid = (ceil(F / 2048), M), block = 256, 8 values per lane.
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t* __restrict__ gu,
                                                       uint16_t* __restrict__ out, int64_t F) {
  const int64_t m = blockIdx.y;
  const int64_t f0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (f0 >= F) return;
  const u32x4_t g8 = *(const u32x4_t*)(gu + m * 2 * F + f0);
  const u32x4_t u8 = *(const u32x4_t*)(gu + m * 2 * F + F + f0);
  u32x4_t o8;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float g = j ? bf16_hi(g8[w]) : bf16_lo(g8[w]);
      const float u = j ? bf16_hi(u8[w]) : bf16_lo(u8[w]);
      const float e = expf(-g);
      const float den = 1.0f + e;
      const float sg = g / den;  // IEEE division
      r[j] = sg * u;
    }
    o8[w] = pack_bf16x2(r[0], r[1]);
  }
  *(u32x4_t*)(out + m * F + f0) = o8;
}

// ---------------------------------------------------------------------------
// Residual add: out = bf16(a + b), 8 values per lane.  grid-stride loop.
__global__ __launch_bounds__(256) void add_kernel(const uint16_t* __restrict__ a,
                                                  const uint16_t* __restrict__ b,
                                                  uint16_t* __restrict__ out, int64_t n8) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8;
       c += (int64_t)gridDim.x * 256) {
    const u32x4_t a8 = ((const u32x4_t*)a)[c];
    const u32x4_t b8 = ((const u32x4_t*)b)[c];
    u32x4_t o8;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o8[w] = pack_bf16x2(bf16_lo(a8[w]) + bf16_lo(b8[w]), bf16_hi(a8[w]) + bf16_hi(b8[w]));
    ((u32x4_t*)out)[c] = o8;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static int last_status() { return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP; }

int launch_embed(const int32_t* tokens, const uint16_t* table, uint16_t* out, int64_t M,
                 int64_t V, int64_t H, hipStream_t stream) {
  hipLaunchKernelGGL(embed_kernel, dim3((unsigned)M), dim3(256), 0, stream, tokens, table, out,
                     V, H);
  return last_status();
}

int rope_table_host(double theta, int D, int64_t max_pos, float* cos_t, float* sin_t) {
  const int half = D / 2;
  for (int64_t p = 0; p < max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double angle = (double)p * pow(theta, -2.0 * (double)i / (double)D);
      cos_t[p * half + i] = (float)cos(angle);
      sin_t[p * half + i] = (float)sin(angle);
    }
  return BI_OK;
}

int launch_rope(const uint16_t* x, int64_t x_stride, uint16_t* out, const int32_t* pos,
                const float* cos_t, const float* sin_t, int64_t M, int heads, int64_t max_pos,
                hipStream_t stream) {
  hipLaunchKernelGGL(rope_kernel, dim3((unsigned)M, (unsigned)((heads + 15) / 16)), dim3(256), 0,
                     stream, x, x_stride, out, pos, cos_t, sin_t, heads, max_pos);
  return last_status();
}

int launch_kv_append(const uint16_t* k, int64_t k_stride, const uint16_t* v, int64_t v_stride,
                     uint16_t* kv, const int32_t* block_table, const int32_t* pos, int64_t M,
                     int Hkv, int max_blocks, int64_t num_pages, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)M, (unsigned)Hkv), dim3(32), 0, stream, k,
                     k_stride, v, v_stride, kv, block_table, pos, Hkv, max_blocks, num_pages);
  return last_status();
}

int launch_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t F,
                    hipStream_t stream) {
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((F + 2047) / 2048), (unsigned)M),
                     dim3(256), 0, stream, gu, out, F);
  return last_status();
}

int launch_add(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
               hipStream_t stream) {
  const int64_t n8 = n / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0,
                     stream, a, b, out, n8);
  return last_status();
}

}  // namespace bi
