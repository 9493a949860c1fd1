// Compacted sparse store (KV Cache reuse page 2: the Index-Aware Cache Layout
// re-packs the selected tokens' KV into a compact block, and only that block is
// loaded; 2.1: blocks aligned to 256 bytes and padded to a power of two).
//
// The store of a (sequence, kv-head) is its valid selected cold tokens in
// selection order (masked and out-of-range entries skipped, duplicates kept),
// cut into units of 64 tokens.  A unit is a K tile and a V tile in exactly the
// chunk layouts of a cold block (2 x tile bytes: 16 KiB for 8-bit codes at
// head_dim 128, a power of two), so the decode streams it like a dense block;
// each token keeps its own block's K and V scales (float2 per token, stored
// beside the units), and the count of stored tokens is kept per (sequence,
// kv-head).
//
//   sparse_compact_kernel  one workgroup per (unit, kv-head, sequence): every
//                          workgroup of a (sequence, kv-head) scans the whole
//                          selection (at most 512 entries) for its tokens'
//                          positions, then copies their K chunks (16 bytes per
//                          token and chunk, unchanged) and assembles every V
//                          chunk of the unit from the tokens' value elements.
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr int kCompactThreads = 256;

// Exclusive prefix sum of v over the workgroup; *total receives the sum.
__device__ __forceinline__ int wg_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kCompactThreads / 64; ++i) {
    before += i < w ? wsum[i] : 0;
    all += wsum[i];
  }
  *total = all;
  return before + x - v;
}

// Stored value element of a row past the count: code 0 (8-bit offset binary 0x80, 4-bit offset
// binary 0x8), fp16 0.
template <int BITS>
constexpr uint32_t zero_elem() { return BITS == 8 ? 0x80u : BITS == 4 ? 8u : 0u; }

template <int D, int BITS>
__global__ __launch_bounds__(kCompactThreads) void sparse_compact_kernel(CompactParams p) {
  using F = Fmt<BITS>;
  constexpr int S = kBlockSize;
  constexpr int E = F::kElems;
  constexpr int TB = F::template tile_bytes<D>();
  constexpr int PER = kMaxTopK / kCompactThreads;  // selection entries per thread
  __shared__ int wsum[kCompactThreads / 64];
  __shared__ int src_phys[S];
  __shared__ int src_row[S];
  const CacheView& c = p.c;
  const int u = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int H = c.H;
  const int bh = b * H + h;
  const int tid = threadIdx.x;
  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  // ---- positions of the valid entries (selection order)
  const int32_t* sel = p.sel + static_cast<size_t>(bh) * p.k_sel;
  int phys_e[PER], row_e[PER];
  int nvalid = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;  // each thread owns PER consecutive entries: positions stay in order
    const int idx = i < p.k_sel ? sel[i] : -1;
    int ph = -1;
    if (idx >= 0 && idx < sg.n_cold) {
      const int j = idx / S;
      if (j < c.max_blocks) {
        const int hv = c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
        if (hv >= 0 && hv < c.num_phys) ph = hv;
      }
    }
    phys_e[k] = ph;
    row_e[k] = idx % S;
    nvalid += ph >= 0 ? 1 : 0;
  }
  if (tid < S) src_phys[tid] = -1;
  int total;
  int pos = wg_exclusive_scan(nvalid, wsum, &total);  // (its barrier also orders the clear above)
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (phys_e[k] < 0) continue;
    const int r = pos - u * S;
    if (r >= 0 && r < S) {
      src_phys[r] = phys_e[k];
      src_row[r] = row_e[k];
    }
    ++pos;
  }
  if (u == 0 && tid == 0) p.counts[bh] = total;
  __syncthreads();
  const size_t unit = static_cast<size_t>(bh) * p.units + u;
  // ---- per-token scales
  if (tid < S) {
    const int ph = src_phys[tid];
    float2 sc = make_float2(0.f, 0.f);
    if (ph >= 0) sc = *reinterpret_cast<const float2*>(c.scales + (static_cast<size_t>(ph) * H + h) * 2);
    p.scales[unit * S + tid] = sc;
  }
  int8_t* dst = p.units_base + unit * 2 * TB;
  // ---- K chunks: chunk (kc, r) of the unit is chunk (kc, row) of the token's own tile
  for (int vi = tid; vi < (D / E) * S; vi += kCompactThreads) {
    const int kc = vi / S, r = vi % S;
    const int ph = src_phys[r];
    uint4 v;
    if (ph >= 0) {
      const int8_t* src = c.cold + tile_offset(ph, h, 0, H, TB);
      v = reinterpret_cast<const uint4*>(src)[kc * S + src_row[r]];
    } else {
      const uint32_t z = BITS == 8 ? 0x80808080u : zero_elem<BITS>() * 0x11111111u;
      v = make_uint4(z, z, z, z);
    }
    reinterpret_cast<uint4*>(dst)[vi] = v;
  }
  // ---- V chunks: chunk (vc, ch) holds tokens vc*E .. vc*E + E - 1 of channel ch, gathered one element
  // per token from the tokens' own V tiles
  for (int vi = tid; vi < (S / E) * D; vi += kCompactThreads) {
    const int vc = vi / D, ch = vi % D;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int r = vc * E + e;
      const int ph = src_phys[r];
      const int t = src_row[r];
      uint32_t x = zero_elem<BITS>();
      if (ph >= 0) {
        const int8_t* vt = c.cold + tile_offset(ph, h, 1, H, TB) + ((t / E) * D + ch) * 16;
        if constexpr (BITS == 8) x = static_cast<uint8_t>(vt[t % E]);
        else if constexpr (BITS == 4) x = (static_cast<uint8_t>(vt[nib_byte(t % E)]) >> nib_shift(t % E)) & 0xFu;
        else x = *reinterpret_cast<const uint16_t*>(vt + (t % E) * 2);
      }
      if constexpr (BITS == 8) w[e / 4] |= x << (8 * (e % 4));
      else if constexpr (BITS == 4) w[e / 8] |= x << (8 * (e & 3) + nib_shift(e));  // planar word (nib_byte)
      else w[e / 2] |= x << (16 * (e % 2));
    }
    reinterpret_cast<uint4*>(dst + TB)[vi] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int BITS>
hipError_t launch_compact_db(const CompactParams& p, const LaunchCtx& ctx) {
  const dim3 grid(p.units, p.c.H, p.c.B);
  if (ctx.start) {
    hipExtLaunchKernelGGL(sparse_compact_kernel<D, BITS>, grid, dim3(kCompactThreads), 0, ctx.stream, ctx.start,
                          ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL((sparse_compact_kernel<D, BITS>), grid, dim3(kCompactThreads), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_compact_d(const CompactParams& p, const LaunchCtx& ctx) {
  switch (p.c.bits) {
    case 8: return launch_compact_db<D, 8>(p, ctx);
    case 4: return launch_compact_db<D, 4>(p, ctx);
    case 0: return launch_compact_db<D, 0>(p, ctx);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

hipError_t launch_compact(const CompactParams& p, const LaunchCtx& ctx) {
  return p.c.D == 128 ? detail::launch_compact_d<128>(p, ctx) : detail::launch_compact_d<64>(p, ctx);
}

}  // namespace hkv
