// qg_gemm for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc): the same product, the same
// kernels and the same tile / split choice as qg_gemm, with the workspace taken from a
// fixed device array of this library instead of the caller.
//
// Every split over K the selector makes keeps (slices x workgroup tiles) within one
// workgroup per CU, so its fp32 partials take at most 256 tiles x 128 rows x 256
// columns x 4 bytes = 32 MiB: the array holds that much, and no dense call needs more.
#include <mutex>

#include "qg.h"
#include "qg_device.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;

// One copy per GPU, kept until the process ends.  In host code this name is only a
// stand-in for the symbol: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];

// Device address of this device's scratch array, looked up once per device with that
// device current; nullptr on error.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_ptr[dev] = ptr;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t qg_noalloc_scratch_bytes(void) { return kScratchBytes; }

qg_status qg_gemm_noalloc(const qg_prepared* p, const void* x, const void* x_scale, void* y, int64_t m,
                          void* stream) {
  const size_t need = qg_workspace_bytes(p, m, 0);   // 0 for an invalid handle: qg_gemm then says why
  if (need == 0) return qg_gemm(p, x, x_scale, y, m, nullptr, 0, stream);
  void* ws = scratch_ptr();
  if (!ws) return QG_ERR_HIP;
  // beyond the array the workspace is refused by qg_gemm (QG_ERR_WORKSPACE, before any launch)
  return qg_gemm(p, x, x_scale, y, m, ws, kScratchBytes, stream);
}

}  // extern "C"
