// bi_internal.h -- launchers shared between the kernel files and the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "bi.h"

namespace bi {

// bi_gemm's argument checks (bi_api.hip): BI_OK or the status bi_gemm returns
int check_gemm_args(const void* x, const void* W, const void* y, int64_t M, int64_t N, int64_t K);

// GEMM (bi_gemm.hip)
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool fast, int num_cus);
int64_t fast_split_kc(int64_t M, int64_t N, int64_t K, int num_cus);
int launch_gemm(const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M, int64_t N,
                int64_t K, void* ws, size_t ws_bytes, hipStream_t stream, bool fast, int num_cus);

// RMSNorm (bi_rmsnorm.hip)
int launch_rmsnorm(const uint16_t* x, const uint16_t* g, uint16_t* y, int64_t M, int64_t H,
                   float eps, hipStream_t stream, bool fast);
int launch_add_rmsnorm(const uint16_t* a, const uint16_t* b, const uint16_t* g, uint16_t* sum,
                       uint16_t* y, int64_t M, int64_t H, float eps, hipStream_t stream);

// Paged decode attention (bi_attn.hip)
size_t attn_ws_bytes(const bi_attn_desc* d, bool fast, int num_cus);
int launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                const int32_t* ctx_lens, uint16_t* out, const bi_attn_desc* d, void* ws,
                size_t ws_bytes, hipStream_t stream, bool fast, int num_cus);

size_t sample_ws_bytes(int64_t M);
int launch_sample(const uint16_t* logits, int64_t M, int64_t V, const uint64_t* seeds,
                  const uint64_t* steps, const float* temps, int32_t* tokens, void* ws,
                  hipStream_t stream);
int launch_verify_commit(const int32_t* cand, const int32_t* ver, const int32_t* row_start, int R,
                         int rows, int32_t* accepted, int32_t* commit_len, int32_t* fix_token,
                         hipStream_t stream);
int launch_gemm_segments(const uint16_t* x, const uint16_t* W, float* part, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream);
int launch_gemm_fold(const float* part, uint16_t* y, int64_t M, int64_t N, int64_t S,
                     hipStream_t stream);
int launch_prefill_attn(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                        const int32_t* row_start, const int32_t* ctx_lens, uint16_t* out,
                        const bi_attn_desc* d, int requests, int max_rows_per_request, void* ws,
                        size_t ws_bytes, hipStream_t stream);

// Decoder-layer element-wise steps (bi_layer.hip)
int launch_embed(const int32_t* tokens, const uint16_t* table, uint16_t* out, int64_t M,
                 int64_t V, int64_t H, hipStream_t stream);
int rope_table_host(double theta, int D, int64_t max_pos, float* cos_t, float* sin_t);
int launch_rope(const uint16_t* x, int64_t x_stride, uint16_t* out, const int32_t* pos,
                const float* cos_t, const float* sin_t, int64_t M, int heads, int64_t max_pos,
                hipStream_t stream);
int launch_kv_append(const uint16_t* k, int64_t k_stride, const uint16_t* v, int64_t v_stride,
                     uint16_t* kv, const int32_t* block_table, const int32_t* pos, int64_t M,
                     int Hkv, int max_blocks, int64_t num_pages, hipStream_t stream);
int launch_silu_mul(const uint16_t* gu, uint16_t* out, int64_t M, int64_t F,
                    hipStream_t stream);
int launch_add(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n,
               hipStream_t stream);

// Matrix-core-only loop for measured ceilings (bi_ceiling.hip)
int launch_mfma_ceiling(float* out, int64_t iters, int64_t workgroups, hipStream_t stream);
int launch_read_ceiling(const void* p, int64_t bytes, uint32_t* out, hipStream_t stream);

// Schedule constants reported by bi_version().
static constexpr int SCHED_GEMM_KB = 32;
static constexpr int SCHED_GEMM_KC = 512;
static constexpr int SCHED_RMS_LANES = 256;
static constexpr int SCHED_ATTN_CHUNK = 256;
static constexpr int SCHED_ATTN_TILE = 64;

}  // namespace bi
