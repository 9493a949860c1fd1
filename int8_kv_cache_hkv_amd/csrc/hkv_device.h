// Device helpers shared by the libhkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv_internal.h"

namespace hkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Make LDS written by some lanes of this wave visible to the other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

// Signed byte k (0..3) of a packed word, as float (exact).
__device__ __forceinline__ float sbyte(uint32_t w, int k) {
  return static_cast<float>(static_cast<int8_t>(static_cast<uint8_t>(w >> (8 * k))));
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  uint16_t b = static_cast<uint16_t>(w & 0xffffu);
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  uint16_t b = static_cast<uint16_t>(w >> 16);
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Sequence geometry derived from the cached length.
struct SeqGeom {
  int n, n_hot, n_cold, n_blk;
};
__device__ __forceinline__ SeqGeom seq_geom(int n, int T, int S) {
  SeqGeom g;
  g.n = n < 0 ? 0 : n;
  g.n_hot = g.n < T ? g.n : T;
  g.n_cold = g.n - g.n_hot;
  g.n_blk = cdiv(g.n_cold, S);
  return g;
}

// Byte offset of the (phys, head, K|V) tile inside the cold pool.
__device__ __forceinline__ size_t tile_offset(int phys, int h, int kv, int H, int S, int D) {
  return ((static_cast<size_t>(phys) * H + h) * 2 + kv) * static_cast<size_t>(S) * D;
}

}  // namespace hkv
