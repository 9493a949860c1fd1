// Fixed device scratch for hkv_decode_attn_noalloc: callers that cannot
// allocate (code under HIP graph capture, serving loops that forbid
// hipMalloc) get the decode's workspace from one file-scope device array of
// kScratchBytes instead of a workspace argument.  Each GPU holds its own copy
// of the array until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address on the current device comes from hipGetSymbolAddress, taken once
// per device at the first call on that device and kept, and only that
// address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hkv_internal.h"

namespace hkv {

namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ void scratch_clear_kernel(uint4* p, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t scratch_for_device(hipStream_t stream, void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    // the counters must start at zero (every call leaves them at zero again): clear the whole
    // array once, with a fill kernel on the caller's stream, and wait for it unless the stream is
    // being captured (then the clear is part of the captured work and ordered before the decode)
    hipLaunchKernelGGL(scratch_clear_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(ptr),
                       kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return e;
    if (cap == hipStreamCaptureStatusNone) {
      e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return e;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace hkv
