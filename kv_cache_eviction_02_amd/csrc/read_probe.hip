// Streaming-read probe for gfx950: a measured HBM read ceiling that the decode
// kernel's bandwidth can be compared with.  It is not part of the H2O path and
// has its own small library (libh2o_probe.so), loaded only by the benchmark.
//
// Every thread streams 16-byte non-temporal loads over a grid-stride range,
// U loads in flight per loop turn, and folds them into an XOR.  The XOR is
// stored only when it equals a fixed constant, so the loads cannot be removed
// and the probe writes (practically) nothing.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr unsigned kMagic = 0x9e3779b9u;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                        unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  unsigned acc = 0;
  // every index read below is < n16
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kMagic) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` bytes (a multiple of 16) at device address src (16-byte
// aligned) with `blocks` workgroups of 256 threads, enqueued on `stream`.
// sink: one device word, written only if the XOR of the data equals a fixed
// constant.  Returns 0, 1 for invalid arguments, 2 for a launch error.
int h2o_probe_read(const void* src, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (!src || !sink || blocks < 1 || blocks > (1 << 20) || bytes % 16 != 0 || ((uintptr_t)src & 15u) != 0)
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(kThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
