// Streaming read probe (measurement aid): the time one launch needs to read a
// buffer once with 16-byte non-temporal loads, the access the decode's cold
// tiles use.  It bounds from below what any kernel that must read the same
// bytes in one launch can reach at that size (launch, first-load latency and
// the drain of every CU's request queue do not shrink with the size).
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr int kProbeUnroll = 4;

// Grid-stride loop, kProbeUnroll independent 16-byte loads in flight per
// thread.  The loaded words are folded into one value that is stored only if
// it equals a sentinel, so no load can be dropped and (practically) nothing is
// written.
__global__ void read_probe_kernel(const uint4* src, size_t n16, uint32_t* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) v[k] = load_stream(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = load_stream(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace detail

hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, int threads, uint32_t* sink,
                             const LaunchCtx& ctx) {
  const size_t n16 = bytes / 16;
  if (ctx.start) {
    hipExtLaunchKernelGGL(detail::read_probe_kernel, dim3(workgroups), dim3(threads), 0, ctx.stream, ctx.start,
                          ctx.stop, 0, static_cast<const uint4*>(src), n16, sink);
  } else {
    hipLaunchKernelGGL(detail::read_probe_kernel, dim3(workgroups), dim3(threads), 0, ctx.stream,
                       static_cast<const uint4*>(src), n16, sink);
  }
  return hipGetLastError();
}

}  // namespace hkv
