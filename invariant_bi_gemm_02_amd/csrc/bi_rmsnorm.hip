// bi_rmsnorm.hip -- y[m,h] = bf16((x[m,h] * r_m) * g[h]),
//                   r_m = 1 / sqrt(sum_h x[m,h]^2 / H + eps), fp32 throughout.
//
// Normalization is one of the reductions whose schedule a dynamic batch
// changes (LLM-42 digest, problem statement; Determinism article, 2.2).  The
// batch-invariant kernel reduces each row in one workgroup with a tree fixed
// by H alone:
//   lane t of 256 sums x^2 left to right over h = 8*(t + 256 i) + j
//   (16-byte loads, j = 0..7 inside a load, i = 0, 1, ...);
//   each 64-lane wave combines with an xor butterfly, offsets 32 .. 1;
//   the four wave sums are added ((w0 + w1) + w2) + w3;
//   ms = ss / H, d = ms + eps, r = 1 / sqrt(d), all correctly rounded.
// The fast twin gives each row one wave when M is large enough to fill the
// chip, which changes the tree (and the bits) with M.
#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

__device__ __forceinline__ float sumsq8(const u32x4_t& v, float a) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = bf16_lo(v[w]);
    const float hi = bf16_hi(v[w]);
    a = a + lo * lo;
    a = a + hi * hi;
  }
  return a;
}

__device__ __forceinline__ u32x4_t scale8(const u32x4_t& xv, const u32x4_t& gv, float r) {
  u32x4_t o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a = (bf16_lo(xv[w]) * r) * bf16_lo(gv[w]);
    const float b = (bf16_hi(xv[w]) * r) * bf16_hi(gv[w]);
    o[w] = pack_bf16x2(a, b);
  }
  return o;
}

// ms, d, sqrt and the reciprocal are each one IEEE correctly rounded
// operation.  (__builtin_sqrtf lowers to the correctly rounded sequence on
// gfx950; the __fsqrt_rn wrapper maps to the approximate native sqrt.)
__device__ __forceinline__ float inv_rms(float ss, int H, float eps) {
  const float ms = ss / (float)H;
  const float d = ms + eps;
  return 1.0f / __builtin_sqrtf(d);
}

// grid = M, block = 256.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ g,
                                                      uint16_t* __restrict__ y, int H, float eps) {
  __shared__ float wsum[4];
  const int t = threadIdx.x;
  const uint16_t* xr = x + (size_t)blockIdx.x * H;
  uint16_t* yr = y + (size_t)blockIdx.x * H;
  float a = 0.0f;
  for (int base = 8 * t; base < H; base += 8 * 256) a = sumsq8(ldg128(xr + base), a);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = a + __shfl_xor(a, o, 64);
  if ((t & 63) == 0) wsum[t >> 6] = a;
  __syncthreads();
  const float ss = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float r = inv_rms(ss, H, eps);
  for (int base = 8 * t; base < H; base += 8 * 256)
    stg128(yr + base, scale8(ldg128(xr + base), ldg128(g + base), r));
}

// The same kernel for rows of at most 8 * 256 * CH values: the row's x and
// the gain are loaded into registers once, before the reduction, and the
// scaling reads them from there (one memory round trip, x read once).  The
// lane sums, tree and scaling are those above, term for term.
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ g,
                                                          uint16_t* __restrict__ y, int H,
                                                          float eps) {
  __shared__ float wsum[4];
  const int t = threadIdx.x;
  const uint16_t* xr = x + (size_t)blockIdx.x * H;
  uint16_t* yr = y + (size_t)blockIdx.x * H;
  u32x4_t xv[CH], gv[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int base = 8 * (t + 256 * i);
    if (base < H) {
      xv[i] = ldg128(xr + base);
      gv[i] = ldg128(g + base);
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    if (8 * (t + 256 * i) < H) a = sumsq8(xv[i], a);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = a + __shfl_xor(a, o, 64);
  if ((t & 63) == 0) wsum[t >> 6] = a;
  __syncthreads();
  const float ss = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float r = inv_rms(ss, H, eps);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int base = 8 * (t + 256 * i);
    if (base < H) stg128(yr + base, scale8(xv[i], gv[i], r));
  }
}

// Fast twin for large M: one wave per row, four rows per workgroup; rows of
// up to 8 * 64 * CH values stay in registers between the two passes (CH = 0:
// any H, read twice).
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_row_per_wave_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ g, uint16_t* __restrict__ y,
    int M, int H, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint16_t* xr = x + (size_t)row * H;
  uint16_t* yr = y + (size_t)row * H;
  float a = 0.0f;
  if constexpr (CH > 0) {
    u32x4_t xv[CH], gv[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int base = 8 * (lane + 64 * i);
      if (base < H) {
        xv[i] = ldg128(xr + base);
        gv[i] = ldg128(g + base);
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (8 * (lane + 64 * i) < H) a = sumsq8(xv[i], a);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = a + __shfl_xor(a, o, 64);
    const float r = inv_rms(a, H, eps);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int base = 8 * (lane + 64 * i);
      if (base < H) stg128(yr + base, scale8(xv[i], gv[i], r));
    }
  } else {
    for (int base = 8 * lane; base < H; base += 8 * 64) a = sumsq8(ldg128(xr + base), a);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) a = a + __shfl_xor(a, o, 64);
    const float r = inv_rms(a, H, eps);
    for (int base = 8 * lane; base < H; base += 8 * 64)
      stg128(yr + base, scale8(ldg128(xr + base), ldg128(g + base), r));
  }
}

// Residual add and the RMSNorm that follows it, in one pass over the row:
// sum = bf16(a + b) (the residual add's arithmetic), then y = RMSNorm(sum)
// with the tree above, reading the bf16 sums from registers.  The same bits
// as the two calls.  grid = M, block = 256; H <= 8 * 256 * ADD_RMS_CHUNKS.
// A lane reads each of its chunks of a and b before writing that chunk of
// sum, so sum may be a or b: a, b and sum are therefore not restrict
// pointers (sum may alias either input); g and y alias nothing.
static constexpr int ADD_RMS_CHUNKS = 4;
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(
    const uint16_t* a, const uint16_t* b, const uint16_t* __restrict__ g,
    uint16_t* sum, uint16_t* __restrict__ y, int H, float eps) {
  __shared__ float wsum[4];
  const int t = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * H;
  u32x4_t s8[ADD_RMS_CHUNKS];
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < ADD_RMS_CHUNKS; ++i) {
    const int base = 8 * (t + 256 * i);
    if (base < H) {
      const u32x4_t a8 = ldg128(a + row + base);
      const u32x4_t b8 = ldg128(b + row + base);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        s8[i][w] = pack_bf16x2(bf16_lo(a8[w]) + bf16_lo(b8[w]), bf16_hi(a8[w]) + bf16_hi(b8[w]));
      stg128(sum + row + base, s8[i]);
      acc = sumsq8(s8[i], acc);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc = acc + __shfl_xor(acc, o, 64);
  if ((t & 63) == 0) wsum[t >> 6] = acc;
  __syncthreads();
  const float ss = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float r = inv_rms(ss, H, eps);
#pragma unroll
  for (int i = 0; i < ADD_RMS_CHUNKS; ++i) {
    const int base = 8 * (t + 256 * i);
    if (base < H) stg128(y + row + base, scale8(s8[i], ldg128(g + base), r));
  }
}

int launch_add_rmsnorm(const uint16_t* a, const uint16_t* b, const uint16_t* g, uint16_t* sum,
                       uint16_t* y, int64_t M, int64_t H, float eps, hipStream_t stream) {
  if (H > 8 * 256 * ADD_RMS_CHUNKS) return BI_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, stream, a, b, g, sum, y,
                     (int)H, eps);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

int launch_rmsnorm(const uint16_t* x, const uint16_t* g, uint16_t* y, int64_t M, int64_t H,
                   float eps, hipStream_t stream, bool fast) {
  if (fast && M >= 1024) {
    const dim3 grid((unsigned)((M + 3) / 4));
    if (H <= 4096)
      hipLaunchKernelGGL(rmsnorm_row_per_wave_kernel<8>, grid, dim3(256), 0, stream, x, g, y,
                         (int)M, (int)H, eps);
    else
      hipLaunchKernelGGL(rmsnorm_row_per_wave_kernel<0>, grid, dim3(256), 0, stream, x, g, y,
                         (int)M, (int)H, eps);
  } else if (H <= 2048) {
    hipLaunchKernelGGL(rmsnorm_reg_kernel<1>, dim3((unsigned)M), dim3(256), 0, stream, x, g, y,
                       (int)H, eps);
  } else if (H <= 4096) {
    hipLaunchKernelGGL(rmsnorm_reg_kernel<2>, dim3((unsigned)M), dim3(256), 0, stream, x, g, y,
                       (int)H, eps);
  } else if (H <= 8192) {
    hipLaunchKernelGGL(rmsnorm_reg_kernel<4>, dim3((unsigned)M), dim3(256), 0, stream, x, g, y,
                       (int)H, eps);
  } else {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, g, y, (int)H,
                       eps);
  }
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
