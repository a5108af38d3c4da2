// bi_api.hip -- the extern "C" entry points declared in include/bi.h:
// argument checks, workspace sizing, status codes and version string.
// Every check happens before anything is enqueued.
#include <math.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "bi_internal.h"

#ifndef BI_GIT_SHA
#define BI_GIT_SHA "unknown"
#endif

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// CU count of the current device, read once per device; only the fast twins
// use it (the batch-invariant entry points never look at it).
// The cache entries are atomics: two threads that race on a device's first
// call both read the same attribute and store the same value.
int current_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int check_gemm(const void* x, const void* W, const void* y, int64_t M, int64_t N, int64_t K) {
  if (!x || !W || !y) return BI_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0) return BI_ERR_SHAPE;
  if (M >= kMaxElems || N >= kMaxElems || K >= kMaxElems) return BI_ERR_SHAPE;
  if (M * K >= kMaxElems || K * N >= kMaxElems || M * N >= kMaxElems) return BI_ERR_SHAPE;
  if (K % 32 != 0 || N % 64 != 0) return BI_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W) || !aligned16(y)) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

int check_rms(const void* x, const void* g, const void* y, int64_t M, int64_t H) {
  if (!x || !g || !y) return BI_ERR_NULL;
  if (M <= 0 || H <= 0 || M >= kMaxElems || H >= kMaxElems || M * H >= kMaxElems)
    return BI_ERR_SHAPE;
  if (H % 8 != 0) return BI_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(g) || !aligned16(y)) return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

int check_attn(const void* q, const void* kv, const void* bt, const void* cl, const void* out,
               const bi_attn_desc* d) {
  if (!q || !kv || !bt || !cl || !out || !d) return BI_ERR_NULL;
  if (d->batch <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->page_size <= 0 || d->max_blocks_per_seq <= 0 || d->num_pages <= 0 || d->max_ctx_len <= 0)
    return BI_ERR_SHAPE;
  if ((int64_t)d->max_ctx_len > (int64_t)d->max_blocks_per_seq * d->page_size) return BI_ERR_SHAPE;
  if ((int64_t)d->batch * d->max_blocks_per_seq >= kMaxElems) return BI_ERR_SHAPE;
  if (d->head_dim != 128 || d->page_size != 16) return BI_ERR_UNSUPPORTED;
  if (d->max_ctx_len > 262144) return BI_ERR_UNSUPPORTED;  // 1024 chunks of 256
  if (d->num_q_heads % d->num_kv_heads != 0) return BI_ERR_UNSUPPORTED;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return BI_ERR_UNSUPPORTED;
  if (!(d->scale == d->scale)) return BI_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || ((uintptr_t)bt & 3u) ||
      ((uintptr_t)cl & 3u))
    return BI_ERR_UNSUPPORTED;
  return BI_OK;
}

// A copy of the descriptor with the default softmax scale filled in: a
// scale <= 0 (or -0) selects 1/sqrt(head_dim), the usual attention scale,
// rounded as fp32 sqrt then fp32 division.
bi_attn_desc resolved(const bi_attn_desc* d) {
  bi_attn_desc r = *d;
  if (r.scale <= 0.f) r.scale = 1.0f / sqrtf((float)r.head_dim);
  return r;
}

}  // namespace

namespace bi {
int check_gemm_args(const void* x, const void* W, const void* y, int64_t M, int64_t N, int64_t K) {
  return check_gemm(x, W, y, M, N, K);
}
}  // namespace bi

extern "C" {

const char* bi_version(void) {
  static char buf[512];
  static std::once_flag once;
  std::call_once(once, [] {
    snprintf(buf, sizeof buf,
             "libbi 0.1.0 git=%s hip=%d.%d target=gfx950 "
             "gemm: mfma_f32_16x16x32_bf16 KB=%d KC=%d fold=left skinny_maxM=64 "
             "tile=256x128 whole_rounds=256x192 last_partial_round=128x128 "
             "fold128_below=192tiles fold64_below=192tiles128 "
             "slice_below=192tiles64; "
             "rmsnorm: lanes=%d vec=8 butterfly=32..1 waves=((0+1)+2)+3 sqrt/div=IEEE; "
             "attn: chunk=%d tile=%d qk=mfma16x16x32 combine=chunk-order exp=__expf",
             BI_GIT_SHA, HIP_VERSION_MAJOR, HIP_VERSION_MINOR, bi::SCHED_GEMM_KB, bi::SCHED_GEMM_KC,
             bi::SCHED_RMS_LANES, bi::SCHED_ATTN_CHUNK, bi::SCHED_ATTN_TILE);
  });
  return buf;
}

const char* bi_status_string(int status) {
  switch (status) {
    case BI_OK: return "ok";
    case BI_ERR_NULL: return "null pointer";
    case BI_ERR_SHAPE: return "bad shape";
    case BI_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case BI_ERR_WORKSPACE: return "workspace too small";
    case BI_ERR_HIP: return "HIP launch failed";
    case BI_ERR_SCRATCH: return "needs more scratch than the library's static array holds";
    default: return "unknown status";
  }
}

size_t bi_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return bi::gemm_ws_bytes(M, N, K, false, 0);
}

size_t bi_gemm_fast_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return bi::gemm_ws_bytes(M, N, K, true, current_cus());
}

static int gemm_entry(const bi_bf16* x, const bi_bf16* W, bi_bf16* y, int64_t M, int64_t N,
                      int64_t K, void* ws, size_t ws_bytes, void* stream, bool fast) {
  int st = check_gemm(x, W, y, M, N, K);
  if (st != BI_OK) return st;
  const int cus = fast ? current_cus() : 0;
  const size_t need = bi::gemm_ws_bytes(M, N, K, fast, cus);
  if (need > 0 && (!ws || ws_bytes < need)) return BI_ERR_WORKSPACE;
  if (ws && !aligned16(ws)) return BI_ERR_UNSUPPORTED;
  return bi::launch_gemm(x, W, y, M, N, K, ws, ws_bytes, (hipStream_t)stream, fast, cus);
}

int bi_gemm(const bi_bf16* x, const bi_bf16* W, bi_bf16* y, int64_t M, int64_t N, int64_t K,
            void* ws, size_t ws_bytes, void* stream) {
  return gemm_entry(x, W, y, M, N, K, ws, ws_bytes, stream, false);
}

int bi_gemm_fast(const bi_bf16* x, const bi_bf16* W, bi_bf16* y, int64_t M, int64_t N, int64_t K,
                 void* ws, size_t ws_bytes, void* stream) {
  return gemm_entry(x, W, y, M, N, K, ws, ws_bytes, stream, true);
}

int bi_gemm_segments(const bi_bf16* x, const bi_bf16* W, float* part, int64_t M, int64_t N,
                     int64_t K, void* stream) {
  int st = check_gemm(x, W, part, M, N, K);
  if (st != BI_OK) return st;
  const int64_t S = (K + 511) / 512;
  if (S * M * N >= kMaxElems * 64) return BI_ERR_SHAPE;
  return bi::launch_gemm_segments(x, W, part, M, N, K, (hipStream_t)stream);
}

int bi_gemm_fold(const float* part, bi_bf16* y, int64_t M, int64_t N, int64_t S, void* stream) {
  if (!part || !y) return BI_ERR_NULL;
  if (M <= 0 || N <= 0 || S <= 0 || M > 65535 || S > 65535 || N >= kMaxElems ||
      M * N >= kMaxElems)
    return BI_ERR_SHAPE;
  if (N % 64 != 0 || !aligned16(part) || !aligned16(y)) return BI_ERR_UNSUPPORTED;
  return bi::launch_gemm_fold(part, y, M, N, S, (hipStream_t)stream);
}

size_t bi_sample_workspace_bytes(int64_t M) { return M > 0 ? bi::sample_ws_bytes(M) : 0; }

int bi_sample(const bi_bf16* logits, int64_t M, int64_t V, const uint64_t* seeds,
              const uint64_t* steps, const float* temperature, int32_t* tokens, void* ws,
              size_t ws_bytes, void* stream) {
  if (!logits || !seeds || !steps || !temperature || !tokens) return BI_ERR_NULL;
  if (M <= 0 || V <= 0 || M > 65535 || V >= kMaxElems || M * V >= kMaxElems * 64)
    return BI_ERR_SHAPE;
  if (((uintptr_t)logits & 1u) || ((uintptr_t)seeds & 7u) || ((uintptr_t)steps & 7u) ||
      ((uintptr_t)temperature & 3u) || ((uintptr_t)tokens & 3u))
    return BI_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < bi::sample_ws_bytes(M)) return BI_ERR_WORKSPACE;
  if ((uintptr_t)ws & 3u) return BI_ERR_UNSUPPORTED;
  return bi::launch_sample(logits, M, V, seeds, steps, temperature, tokens, ws,
                           (hipStream_t)stream);
}

int bi_verify_commit(const int32_t* candidates, const int32_t* verified, int32_t rows,
                     const int32_t* row_start, int32_t requests, int32_t* accepted,
                     int32_t* commit_len, int32_t* fix_token, void* stream) {
  if (!candidates || !verified || !row_start || !accepted || !commit_len || !fix_token)
    return BI_ERR_NULL;
  if (rows < 0 || requests <= 0) return BI_ERR_SHAPE;
  if (((uintptr_t)candidates | (uintptr_t)verified | (uintptr_t)row_start | (uintptr_t)accepted |
       (uintptr_t)commit_len | (uintptr_t)fix_token) & 3u)
    return BI_ERR_UNSUPPORTED;
  return bi::launch_verify_commit(candidates, verified, row_start, requests, rows, accepted,
                                  commit_len, fix_token, (hipStream_t)stream);
}

int bi_rmsnorm(const bi_bf16* x, const bi_bf16* g, bi_bf16* y, int64_t M, int64_t H, float eps,
               void* stream) {
  int st = check_rms(x, g, y, M, H);
  if (st != BI_OK) return st;
  return bi::launch_rmsnorm(x, g, y, M, H, eps, (hipStream_t)stream, false);
}

int bi_rmsnorm_fast(const bi_bf16* x, const bi_bf16* g, bi_bf16* y, int64_t M, int64_t H,
                    float eps, void* stream) {
  int st = check_rms(x, g, y, M, H);
  if (st != BI_OK) return st;
  return bi::launch_rmsnorm(x, g, y, M, H, eps, (hipStream_t)stream, true);
}

int bi_add_rmsnorm(const bi_bf16* a, const bi_bf16* b, const bi_bf16* g, bi_bf16* sum,
                   bi_bf16* y, int64_t M, int64_t H, float eps, void* stream) {
  if (!a || !b || !sum) return BI_ERR_NULL;
  int st = check_rms(a, g, y, M, H);
  if (st != BI_OK) return st;
  if (!aligned16(b) || !aligned16(sum)) return BI_ERR_UNSUPPORTED;
  return bi::launch_add_rmsnorm(a, b, g, sum, y, M, H, eps, (hipStream_t)stream);
}

size_t bi_attn_workspace_bytes(const bi_attn_desc* d) {
  if (!d || d->batch <= 0 || d->num_q_heads <= 0 || d->max_ctx_len <= 0) return 0;
  return bi::attn_ws_bytes(d, false, 0);
}

size_t bi_attn_fast_workspace_bytes(const bi_attn_desc* d) {
  if (!d || d->batch <= 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->max_ctx_len <= 0)
    return 0;
  return bi::attn_ws_bytes(d, true, current_cus());
}

static int attn_entry(const bi_bf16* q, const bi_bf16* kv, const int32_t* bt, const int32_t* cl,
                      bi_bf16* out, const bi_attn_desc* d, void* ws, size_t ws_bytes,
                      void* stream, bool fast) {
  int st = check_attn(q, kv, bt, cl, out, d);
  if (st != BI_OK) return st;
  const int cus = fast ? current_cus() : 0;
  const size_t need = bi::attn_ws_bytes(d, fast, cus);
  if (!ws || ws_bytes < need) return BI_ERR_WORKSPACE;
  if (!aligned16(ws)) return BI_ERR_UNSUPPORTED;
  const bi_attn_desc dd = resolved(d);
  return bi::launch_attn(q, kv, bt, cl, out, &dd, ws, ws_bytes, (hipStream_t)stream, fast, cus);
}

int bi_paged_decode_attn(const bi_bf16* q, const bi_bf16* kv_pages, const int32_t* block_table,
                         const int32_t* ctx_lens, bi_bf16* out, const bi_attn_desc* d, void* ws,
                         size_t ws_bytes, void* stream) {
  return attn_entry(q, kv_pages, block_table, ctx_lens, out, d, ws, ws_bytes, stream, false);
}

int bi_paged_decode_attn_fast(const bi_bf16* q, const bi_bf16* kv_pages,
                              const int32_t* block_table, const int32_t* ctx_lens, bi_bf16* out,
                              const bi_attn_desc* d, void* ws, size_t ws_bytes, void* stream) {
  return attn_entry(q, kv_pages, block_table, ctx_lens, out, d, ws, ws_bytes, stream, true);
}

int bi_paged_prefill_attn(const bi_bf16* q, const bi_bf16* kv_pages, const int32_t* block_table,
                          const int32_t* row_start, const int32_t* ctx_lens, bi_bf16* out,
                          const bi_attn_desc* d, int32_t requests, int32_t max_rows_per_request,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!row_start) return BI_ERR_NULL;
  int st = check_attn(q, kv_pages, block_table, ctx_lens, out, d);
  if (st != BI_OK) return st;
  if (requests <= 0 || max_rows_per_request <= 0 || max_rows_per_request > d->batch)
    return BI_ERR_SHAPE;
  if ((int64_t)requests * d->max_blocks_per_seq >= kMaxElems) return BI_ERR_SHAPE;
  if ((uintptr_t)row_start & 3u) return BI_ERR_UNSUPPORTED;
  const size_t need = bi::attn_ws_bytes(d, false, 0);
  if (!ws || ws_bytes < need) return BI_ERR_WORKSPACE;
  if (!aligned16(ws)) return BI_ERR_UNSUPPORTED;
  const bi_attn_desc dd = resolved(d);
  return bi::launch_prefill_attn(q, kv_pages, block_table, row_start, ctx_lens, out, &dd, requests,
                                 max_rows_per_request, ws, ws_bytes, (hipStream_t)stream);
}

int bi_embed(const int32_t* tokens, const bi_bf16* table, bi_bf16* out, int64_t M, int64_t V,
             int64_t H, void* stream) {
  if (!tokens || !table || !out) return BI_ERR_NULL;
  if (M <= 0 || V <= 0 || H <= 0 || M >= kMaxElems || V * H >= ((int64_t)1 << 40) ||
      M * H >= kMaxElems)
    return BI_ERR_SHAPE;
  if (H % 8 != 0 || !aligned16(table) || !aligned16(out) || ((uintptr_t)tokens & 3u))
    return BI_ERR_UNSUPPORTED;
  return bi::launch_embed(tokens, table, out, M, V, H, (hipStream_t)stream);
}

int bi_rope_table(double theta, int32_t head_dim, int64_t max_pos, float* cos_t, float* sin_t) {
  if (!cos_t || !sin_t) return BI_ERR_NULL;
  if (!(theta > 0.0) || head_dim < 2 || head_dim % 2 != 0 || max_pos <= 0 ||
      max_pos * head_dim >= kMaxElems)
    return BI_ERR_SHAPE;
  return bi::rope_table_host(theta, head_dim, max_pos, cos_t, sin_t);
}

int bi_rope(const bi_bf16* x, int64_t x_row_stride, bi_bf16* out, const int32_t* pos,
            const float* cos_t, const float* sin_t, int64_t M, int32_t heads, int32_t head_dim,
            int64_t max_pos, void* stream) {
  if (!x || !out || !pos || !cos_t || !sin_t) return BI_ERR_NULL;
  if (M <= 0 || heads <= 0 || max_pos <= 0 || M >= kMaxElems || heads > 65535 ||
      x_row_stride < (int64_t)heads * 128 || M * x_row_stride >= kMaxElems)
    return BI_ERR_SHAPE;
  if (head_dim != 128 || ((uintptr_t)x & 7u) || ((uintptr_t)out & 7u) || ((uintptr_t)pos & 3u) ||
      (x_row_stride & 3) || !aligned16(cos_t) || !aligned16(sin_t))
    return BI_ERR_UNSUPPORTED;
  return bi::launch_rope(x, x_row_stride, out, pos, cos_t, sin_t, M, heads, max_pos,
                         (hipStream_t)stream);
}

int bi_kv_append(const bi_bf16* k, int64_t k_row_stride, const bi_bf16* v, int64_t v_row_stride,
                 bi_bf16* kv_pages, const int32_t* block_table, const int32_t* pos, int64_t M,
                 int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t max_blocks,
                 int64_t num_pages, void* stream) {
  if (!k || !v || !kv_pages || !block_table || !pos) return BI_ERR_NULL;
  if (M <= 0 || num_kv_heads <= 0 || num_kv_heads > 65535 || max_blocks <= 0 ||
      num_pages <= 0 || M >= kMaxElems || M * (int64_t)max_blocks >= kMaxElems ||
      k_row_stride < (int64_t)num_kv_heads * 128 || v_row_stride < (int64_t)num_kv_heads * 128)
    return BI_ERR_SHAPE;
  if (head_dim != 128 || page_size != 16 || k_row_stride % 8 != 0 || v_row_stride % 8 != 0 ||
      !aligned16(k) || !aligned16(v) || !aligned16(kv_pages) || ((uintptr_t)block_table & 3u) ||
      ((uintptr_t)pos & 3u))
    return BI_ERR_UNSUPPORTED;
  return bi::launch_kv_append(k, k_row_stride, v, v_row_stride, kv_pages, block_table, pos, M,
                              num_kv_heads, max_blocks, num_pages, (hipStream_t)stream);
}

int bi_silu_mul(const bi_bf16* gu, bi_bf16* out, int64_t M, int64_t F, void* stream) {
  if (!gu || !out) return BI_ERR_NULL;
  if (M <= 0 || F <= 0 || M > 65535 || M * 2 * F >= kMaxElems) return BI_ERR_SHAPE;
  if (F % 8 != 0 || !aligned16(gu) || !aligned16(out)) return BI_ERR_UNSUPPORTED;
  return bi::launch_silu_mul(gu, out, M, F, (hipStream_t)stream);
}

int bi_add(const bi_bf16* a, const bi_bf16* b, bi_bf16* out, int64_t n, void* stream) {
  if (!a || !b || !out) return BI_ERR_NULL;
  if (n <= 0 || n >= kMaxElems) return BI_ERR_SHAPE;
  if (n % 8 != 0 || !aligned16(a) || !aligned16(b) || !aligned16(out)) return BI_ERR_UNSUPPORTED;
  return bi::launch_add(a, b, out, n, (hipStream_t)stream);
}

}  // extern "C"
