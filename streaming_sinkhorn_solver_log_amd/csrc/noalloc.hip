// noalloc.hip -- sk_sinkhorn_solve_noalloc: the fixed-budget solve for callers
// that cannot allocate device memory or pass a workspace (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation). Its scratch
// is a file-scope device array of kScratchBytes that the loaded code object
// holds on every GPU it runs on until the process ends.
#include <mutex>

#include "flashsk.h"
#include "sk_api.h"

namespace sk {
namespace {

using namespace api;

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

// One copy per device. In host code this name is a host-side stand-in, not a
// device address: kernels take the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SK_ERR_UNSUPPORTED, "device %d is beyond the %d this entry point serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SK_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SK_OK;
}

}  // namespace
}  // namespace sk

using namespace sk;
using namespace sk::api;

extern "C" {

size_t sk_noalloc_scratch_bytes(void) { return kScratchBytes; }

int sk_sinkhorn_solve_noalloc(const void* x, const void* y, int dtype, int64_t n, int64_t m, int64_t d,
                              const float* a, const float* b, double eps, int32_t iters, int mode, uint32_t flags,
                              float* f, float* g, double* cost, void* stream) {
  clear_error();
  int rc = check_common(x, y, dtype, n, m, d, a, b, eps, solve_path(dtype, d));
  if (rc) return rc;
  if (!f || !g || !cost) return fail(SK_ERR_INVALID_ARG, "null output pointer");
  if (iters < 0) return fail(SK_ERR_INVALID_ARG, "iters must be >= 0");
  if (mode != SK_ALTERNATING && mode != SK_SYMMETRIC) return fail(SK_ERR_INVALID_ARG, "mode %d is not SK_ALTERNATING or SK_SYMMETRIC", mode);
  if (flags & ~(SK_WARM_START | SK_NO_CENTER))
    return fail(SK_ERR_INVALID_ARG, "flags 0x%x: only SK_WARM_START and SK_NO_CENTER apply (SK_CHECK_FINITE waits "
                "for the stream)", flags);
  const size_t need = solve_bytes(dtype, n, m, d);
  if (need > kScratchBytes)
    return fail(SK_ERR_UNSUPPORTED,
                "n=%lld m=%lld d=%lld needs %zu bytes of scratch; the allocation-free solve holds %zu "
                "(use sk_sinkhorn_solve with a workspace)",
                (long long)n, (long long)m, (long long)d, need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  return sk_sinkhorn_solve(x, y, dtype, n, m, d, a, b, eps, iters, mode, flags, f, g, cost, ws, kScratchBytes,
                           stream);
}

}  // extern "C"
