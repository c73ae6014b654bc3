// h2o_prefill_no_alloc: the prefill for callers that cannot allocate device
// memory.  Its row statistics and column sums go to a fixed array in the
// library's code object instead of the ctx's scratch; everything else is
// h2o_prefill_with_output (same kernels, same results).
#include <hip/hip_runtime.h>

#include <mutex>

#include "ctx.h"
#include "h2o.h"

// Row log-sum-exp and column sums of the calls on one device: 2 * units *
// round_up(prompt_len, 16) floats at most H2O_NO_ALLOC_SCRATCH_BYTES.  Each
// device the library runs on holds its own copy until the process ends.  In
// host code this name is only a host-side stand-in, never a device address:
// the address comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) float scratch[H2O_NO_ALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
float* g_scratch[kMaxDevices];  // device address of `scratch` per device; null until first asked

// The current device's copy of `scratch`, asked from the runtime once per
// device (with that device current).
h2o_status scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return H2O_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return H2O_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return H2O_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return H2O_OK;
}

}  // namespace

extern "C" h2o_status h2o_prefill_no_alloc(h2o_ctx* ctx, const void* q, const void* k, const void* v,
                                          int32_t prompt_len, float* out, void* stream) {
  const h2o_status st = h2o::check_prefill(ctx, q, k, v, prompt_len, out);
  if (st != H2O_OK) return st;
  const size_t units = (size_t)ctx->cfg.batch * ctx->cfg.heads;
  const size_t stride = ((size_t)prompt_len + 15) / 16 * 16;
  if (2 * units * stride * sizeof(float) > (size_t)H2O_NO_ALLOC_SCRATCH_BYTES) return H2O_ERR_TOO_LARGE;
  float* base = nullptr;
  const h2o_status sa = scratch_address(&base);
  if (sa != H2O_OK) return sa;
  // Every entry is written by the kernels before it is read (one row statistic
  // per prompt row, one column sum per prompt position), so nothing left by an
  // earlier call needs clearing.
  return h2o::run_prefill(ctx, q, k, v, prompt_len, out, base, base + units * stride, (int32_t)stride, stream);
}
