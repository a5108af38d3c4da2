// bi_noalloc.hip -- bi_gemm for callers that cannot allocate device memory:
// code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc.  The segment sums that bi_gemm sends through the caller's
// workspace go to a file-scope device array instead, of a fixed maximum
// size, which every GPU the library runs on holds until the process ends.
//
// The array's name is a host-side stand-in in host code, not a device
// address: its address on the current device is taken once per device with
// hipGetSymbolAddress, and only that pointer is ever handed to a kernel.
// Each device holds its own copy at its own address.
//
// Every call on a device shares that device's array.  It needs no
// initialisation (each call writes every segment sum before the fold reads
// it) and keeps the last call's contents; calls that overlap on one device,
// on any streams, race on it.
#include <mutex>

#include "bi_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // BI_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == BI_NOALLOC_SCRATCH_BYTES, "header and library disagree");

constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // scratch's device address, per device (null until taken)

// The device address of this device's scratch array, or null when the
// device id is out of range or the runtime cannot give it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int bi_gemm_noalloc(const bi_bf16* x, const bi_bf16* W, bi_bf16* y, int64_t M,
                               int64_t N, int64_t K, void* stream) {
  // bi_gemm's argument checks, then the size check, before touching a device
  const int st = bi::check_gemm_args(x, W, y, M, N, K);
  if (st != BI_OK) return st;
  const size_t need = bi_gemm_workspace_bytes(M, N, K);
  if (need > kScratchBytes) return BI_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return BI_ERR_HIP;
  }
  return bi_gemm(x, W, y, M, N, K, ws, need, stream);
}
