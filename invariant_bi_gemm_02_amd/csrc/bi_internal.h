// bi_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "bi.h"

namespace bi {

// GEMM (bi_gemm.hip)
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool fast, int num_cus);
int64_t fast_split_kc(int64_t M, int64_t N, int64_t K, int num_cus);
int launch_gemm(const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M, int64_t N,
                int64_t K, void* ws, size_t ws_bytes, hipStream_t stream, bool fast, int num_cus);

// RMSNorm (bi_rmsnorm.hip)
int launch_rmsnorm(const uint16_t* x, const uint16_t* g, uint16_t* y, int64_t M, int64_t H,
                   float eps, hipStream_t stream, bool fast);

// Paged decode attention (bi_attn.hip)
size_t attn_ws_bytes(const bi_attn_desc* d, bool fast, int num_cus);
int launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                const int32_t* ctx_lens, uint16_t* out, const bi_attn_desc* d, void* ws,
                size_t ws_bytes, hipStream_t stream, bool fast, int num_cus);

// Schedule constants reported by bi_version().
static constexpr int SCHED_GEMM_KB = 32;
static constexpr int SCHED_GEMM_KC = 512;
static constexpr int SCHED_RMS_LANES = 256;
static constexpr int SCHED_ATTN_CHUNK = 256;
static constexpr int SCHED_ATTN_TILE = 64;

}  // namespace bi
