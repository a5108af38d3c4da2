// bi_ceiling.hip -- measurement helpers, not part of any operation's path:
//   a matrix-core-only loop, so that measurements can quote the bf16 rate the
//   chip sustains at the clock it holds under matrix-core load beside the
//   published peak;
//   a streaming read of one buffer, so that a bandwidth-bound kernel can be
//   set beside the time HBM takes to deliver the same bytes with nothing
//   else to do.
//
// Each wave runs `iters` rounds of eight independent chains of
// v_mfma_f32_16x16x32_bf16 (the instruction every GEMM path issues) on
// operands held in registers: no memory traffic, no LDS, no dependence
// between consecutive ops of a round, so the matrix pipe never waits on a
// result.  Each lane writes one float at the end so that nothing is
// optimised away.
#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

static constexpr int CEIL_CHAINS = 8;

__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float* __restrict__ out, int iters,
                                                           float seed) {
  const int lane = threadIdx.x & 63;
  // operands: small bf16 values that stay finite over any number of rounds
  const float v = seed * (1.0f + 0.001f * (float)lane);
  const uint32_t h = f32_to_bf16_bits(v) * 0x10001u;
  const u32x4_t a = u32x4_t{h, h, h, h};
  const u32x4_t b = u32x4_t{h ^ 0x80008000u, h, h, h ^ 0x80008000u};
  f32x4_t acc[CEIL_CHAINS];
#pragma unroll
  for (int c = 0; c < CEIL_CHAINS; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the eight ops of a round are one asm block, so that each accumulator
  // stays in its own registers (left to itself the compiler rotated them
  // through the accumulator file with extra moves every round)
  for (int i = 0; i < iters; ++i) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
          "+v"(acc[6]), "+v"(acc[7])
        : "v"(a), "v"(b));
  }
  // the results of the last round's ops are read below: the hardware
  // interlocks a VALU read of an MFMA result only after the required wait
  // states, which the trailing nops provide
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CEIL_CHAINS; ++c) s = s + ((acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]));
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

int launch_mfma_ceiling(float* out, int64_t iters, int64_t workgroups, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, out,
                     (int)iters, 0.001f);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

// Streaming read: every 16-byte chunk of p[0 .. n16) is loaded once, four
// chunks per lane per round (consecutive lanes on consecutive chunks, 1 KB per
// wave instruction, non-temporal hint), and XOR-ed into a register; each wave
// writes one word, out[4 * blockIdx.x + wave], so that no load is optimised
// away.
static constexpr int READ_UNROLL = 4;
__global__ __launch_bounds__(256) void read_ceiling_kernel(const u32x4_t* __restrict__ p,
                                                           int64_t n16, uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256 * READ_UNROLL;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 256 * READ_UNROLL + threadIdx.x; base < n16;
       base += stride) {
    u32x4_t v[READ_UNROLL];
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n16 ? ldg128_nt(p + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) acc ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

int launch_read_ceiling(const void* p, int64_t bytes, uint32_t* out, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = 256 * READ_UNROLL;
  const int64_t grid = std::min<int64_t>((n16 + per_wg - 1) / per_wg, BI_CEILING_READ_OUT_WORDS / 4);
  hipLaunchKernelGGL(read_ceiling_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const u32x4_t*)p, n16, out);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi

extern "C" int bi_ceiling_read(const void* p, int64_t bytes, uint32_t* out, void* stream) {
  if (!p || !out) return BI_ERR_NULL;
  if (bytes <= 0 || bytes > ((int64_t)1 << 40)) return BI_ERR_SHAPE;
  if (bytes % 16 != 0 || ((uintptr_t)p & 15u) || ((uintptr_t)out & 3u)) return BI_ERR_UNSUPPORTED;
  return bi::launch_read_ceiling(p, bytes, out, (hipStream_t)stream);
}

extern "C" int bi_ceiling_mfma(float* out, int64_t iters, int64_t workgroups, void* stream) {
  if (!out) return BI_ERR_NULL;
  if (iters <= 0 || iters > (1 << 30) || workgroups <= 0 || workgroups > 65535) return BI_ERR_SHAPE;
  if ((uintptr_t)out & 3u) return BI_ERR_UNSUPPORTED;
  return bi::launch_mfma_ceiling(out, iters, workgroups, (hipStream_t)stream);
}
