// Append / spill / quantise kernels (gfx950).
//
// Hybrid KV Cache page, 2.1: the hot zone keeps the full FP16 KV of the most
// recent hot_tokens tokens; older tokens form the cold zone, stored as INT8
// with a block-wise scale (3.1: 4 or 8 bits; 5.2: 0 bits keeps the cold zone
// in FP16).  4.2 (step 2): the non-hot part is quantised.  Scale per (block,
// kv-head, K|V): s = fl32(max|x| / L) with L = 127 (8 bits) or 7 (4 bits);
// code = clamp(rint(fl32(x / s)), -L, L), round half to even.  A partially
// filled block always holds the codes of its current tokens, so every block
// an append touches is re-quantised from FP16 (older tokens of a partial block
// come from the per-sequence tail shadow).  FP16 tiles store the values
// (scale 1).
//
// Two launches, in stream order (multi-block appends; the single-pass
// append_step_kernel below serves appends that touch at most two blocks):
//   append_quant_kernel  one workgroup per (sequence, touched block, kv-head,
//                        K|V): gathers the tile's FP16 rows (tail shadow, hot
//                        ring, new tokens), reduces max|x|, divides and rounds,
//                        and writes the codes in the tile layout the decode
//                        kernels stream, plus the scale and the block header.
//   append_ring_kernel   one workgroup per (sequence, kv-head): copies the new
//                        partial block's FP16 rows into the tail shadow, then
//                        writes the new tokens into the hot ring (after every
//                        read of the slots they replace); the kv-head 0
//                        workgroup publishes seq_len.
// Both take the cached lengths from the host mirror (kernel arguments), so
// their first loads are the rows themselves.
#include <hip/hip_ext.h>

#include <type_traits>

#include "hkv_device.h"

namespace hkv {

namespace detail {

// Stage of one (block, kv-head, K|V) tile in LDS while it is coded: K row-major ([token][channel]),
// V column-major ([channel][token]), the orders of the tiles' chunks; one byte per code, or the
// fp16 value itself.
template <int D, int BITS>
struct TileStage {
  static constexpr int EB = BITS == 0 ? 2 : 1;
  static constexpr int KROW = D * EB + 16;            // padded K row (bytes)
  static constexpr int VROW = kBlockSize * EB + 16;   // padded V row (bytes)
  static constexpr int BYTES = (kBlockSize * KROW > D * VROW) ? kBlockSize * KROW : D * VROW;
};

// Element i of a row slice held as fp16 pairs (u32x4_t vectors).
template <int NV>
__device__ __forceinline__ uint32_t slice_half_bits(const u32x4_t (&x)[NV], int e) {
  const uint32_t wd = x[e / 8][(e % 8) / 2];
  return (e & 1) ? (wd >> 16) : (wd & 0xffffu);
}

// Stage the CPT elements of token t at channels [c0, c0 + CPT) of one tile: 8-/4-bit codes under
// scale s (rint(fl32(x / s)): every x lies inside the tile's maximum, so |code| <= L without a
// clamp), or the fp16 values.  kv selects the stage order.  With want_err, returns the largest
// |x - code * s| of these elements (fma: the exact difference rounded once to fp32); else 0.
template <int D, int BITS, int CPT, int NV>
__device__ __forceinline__ float stage_row(int8_t* stage, const u32x4_t (&x)[NV], float s, int kv, int t, int c0,
                                           bool want_err) {
  using TS = TileStage<D, BITS>;
  if constexpr (BITS == 0) {
    if (kv == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(stage + t * TS::KROW + c0 * 2);
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[4 * v + i] = x[v][i];
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e)
        *reinterpret_cast<uint16_t*>(stage + (c0 + e) * TS::VROW + 2 * t) = static_cast<uint16_t>(slice_half_bits(x, e));
    }
    return 0.f;
  } else {
    const float rs = quant_recip(s);
    uint32_t q[CPT / 4];
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) {
      uint32_t cb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * i + k;
        const uint32_t wd = x[e / 8][(e % 8) / 2];
        cb[k] = code_bits(quant_quotient((e & 1) ? half_hi(wd) : half_lo(wd), s, rs));
      }
      q[i] = pack_low_bytes(cb[0], cb[1], cb[2], cb[3]);
    }
    float err = 0.f;
    if (want_err) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const uint32_t wd = x[e / 8][(e % 8) / 2];
        const float xv = (e & 1) ? half_hi(wd) : half_lo(wd);
        const float qv = static_cast<float>(static_cast<int8_t>(q[e / 4] >> (8 * (e % 4))));
        err = fmaxf(err, __builtin_fabsf(fmaf(-qv, s, xv)));
      }
    }
    if (kv == 0) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(stage + t * TS::KROW + c0);
#pragma unroll
      for (int i = 0; i < CPT / 4; ++i) dst[i] = q[i];
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e) stage[(c0 + e) * TS::VROW + t] = static_cast<int8_t>(q[e / 4] >> (8 * (e % 4)));
    }
    return err;
  }
}

// Stage a V tile's elements held as NV tokens (tg NV + r, r < NV) x 8 channels [c0, c0 + 8): the
// tile is channel-major, so each channel's NV codes (or fp16 values) are adjacent in the stage and
// leave in one store.  Codes, the error and want_err as in stage_row.
template <int D, int BITS, int NV>
__device__ __forceinline__ float stage_cols(int8_t* stage, const u32x4_t (&x)[NV], float s, int tg, int c0,
                                            bool want_err) {
  using TS = TileStage<D, BITS>;
  static_assert(NV == 2 || NV == 4, "2 or 4 tokens per thread");
  if constexpr (BITS == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t hv[NV];
#pragma unroll
      for (int r = 0; r < NV; ++r) hv[r] = (e & 1) ? (x[r][e / 2] >> 16) : (x[r][e / 2] & 0xffffu);
      int8_t* dst = stage + (c0 + e) * TS::VROW + tg * NV * 2;
      if constexpr (NV == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
      } else {
        *reinterpret_cast<uint32_t*>(dst) = hv[0] | (hv[1] << 16);
      }
    }
    return 0.f;
  } else {
    const float rs = quant_recip(s);
    float err = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {  // channel c0 + e: its NV codes, packed and stored together
      uint32_t cb[NV];
#pragma unroll
      for (int r = 0; r < NV; ++r) {
        const uint32_t wd = x[r][e / 2];
        const float xv = (e & 1) ? half_hi(wd) : half_lo(wd);
        cb[r] = code_bits(quant_quotient(xv, s, rs));
        if (want_err) err = fmaxf(err, __builtin_fabsf(fmaf(-static_cast<float>(static_cast<int8_t>(cb[r])), s, xv)));
      }
      int8_t* dst = stage + (c0 + e) * TS::VROW + tg * NV;
      if constexpr (NV == 4) {
        *reinterpret_cast<uint32_t*>(dst) = pack_low_bytes(cb[0], cb[1], cb[2], cb[3]);
      } else {
        *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>((cb[0] & 0xffu) | ((cb[1] & 0xffu) << 8));
      }
    }
    return err;
  }
}

// Largest value of v over the workgroup (every thread calls it; red holds kWaves floats).
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_dpp(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[w]);
  return r;
}

// Largest |x - code * s| over a row slice coded with scale s (8-bit codes; the codes are recomputed).
template <int NV>
__device__ __forceinline__ float slice_err8(const u32x4_t (&x)[NV], float s) {
  if (!(s > 0.f)) return 0.f;
  const float rs = quant_recip(s);
  float err = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = half_lo(x[v][i]), b = half_hi(x[v][i]);
      err = fmaxf(err, __builtin_fabsf(fmaf(-quant_code<127>(a, s, rs), s, a)));
      err = fmaxf(err, __builtin_fabsf(fmaf(-quant_code<127>(b, s, rs), s, b)));
    }
  return err;
}

// Write a whole staged tile in its chunk layout (16-byte vectors, coalesced).
template <int D, int BITS>
__device__ __forceinline__ void write_tile(int8_t* tile, const int8_t* stage, int kv, int tid) {
  using TS = TileStage<D, BITS>;
  constexpr int S = kBlockSize;
  constexpr int E = Fmt<BITS>::kElems;
  constexpr int NVEC = Fmt<BITS>::template tile_bytes<D>() / 16;
  for (int vi = tid; vi < NVEC; vi += kThreads) {
    uint4 out;
    if (kv == 0) {
      const int kc = vi / S, tt = vi % S;  // chunk (kc, tt): elements [kc E, kc E + E) of token tt
      out = chunk_from_stage<BITS>(stage + tt * TS::KROW + kc * E * TS::EB);
    } else {
      const int vc = vi / D, cc = vi % D;  // chunk (vc, cc): tokens [vc E, vc E + E) of channel cc
      out = chunk_from_stage<BITS>(stage + cc * TS::VROW + vc * E * TS::EB);
    }
    reinterpret_cast<uint4*>(tile)[vi] = out;
  }
}

// Scale of a tile whose largest magnitude is m: fl32(m / L) (IEEE fp32 division), or 1 for fp16 tiles.
template <int BITS>
__device__ __forceinline__ float tile_scale(float m) {
  if constexpr (BITS == 0) return 1.f;
  else return m / static_cast<float>(Fmt<BITS>::kLimit);
}

// One workgroup per (sequence, touched block, kv-head, K|V): one tile, so that the K and V tiles of a
// block are coded side by side rather than one after the other.
template <int D, int BITS>
__global__ __launch_bounds__(kThreads) void append_quant_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int TPT = kThreads / S;     // threads per token row
  constexpr int CPT = D / TPT;          // channels per thread (32 or 16)
  constexpr int NV = CPT / 8;           // 16-byte vectors per thread and row
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  __shared__ __align__(16) int8_t stage[TileStage<D, BITS>::BYTES];
  __shared__ float red[kWaves];
  __shared__ float rerr[kWaves];

  const CacheView& c = p.c;
  const int H = c.H, T = c.T;
  const int kv = blockIdx.x & 1;
  const int wg = blockIdx.x >> 1;
  const int h = wg % H;
  const int rest = wg / H;
  const int jj = rest % p.touched_max;
  const int bl = rest / p.touched_max;
  if (bl >= p.n_seq) return;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  if (nn <= 0) return;
  const int n0 = p.n0[bl];  // the host mirror: no load before the rows are requested
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  if (cold1 <= cold0) return;
  const int j = cold0 / S + jj;
  if (j * S >= cold1 || j >= c.max_blocks) return;
  hkv_block_header* hdr = c.headers + static_cast<size_t>(b) * c.max_blocks + j;
  const int ph_lane = hdr->phys_block;  // resolved only before the writes (its wait would hold the row loads)
  const int valid = min(S, cold1 - j * S);

  const int tid = threadIdx.x;
  // K tiles (token-major): thread = (token t, channel slice part), NV vectors of 8 channels of token
  // t.  V tiles (channel-major): thread = (token group tg, channel group cg), vector r = 8 channels of
  // token tg NV + r, so that the stage takes each channel's NV codes in one store.
  constexpr int NTG = S / NV;           // token groups of a V tile
  static_assert(NTG * (D / 8) == kThreads, "a V tile is NV tokens x 8 channels per thread");
  const int t = tid / TPT;              // (K) token row inside the block
  const int part = tid % TPT;           // (K) channel slice
  const int tg = tid % NTG;             // (V) token group
  const int cg = tid / NTG;             // (V) channel group

  // ---- the FP16 row slices: the tail shadow (rows of a partial block already cached), the hot
  // ring (rows leaving it) or the new tokens
  u32x4_t x[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int tok = kv ? tg * NV + v : t;
    const int col = kv ? cg * 8 : part * CPT + 8 * v;
    const int pos = j * S + tok;
    const _Float16* row = nullptr;
    if (tok < valid) {
      if (pos < cold0) {
        row = c.tail + ((static_cast<size_t>(b) * H + h) * 2 + kv) * S * D + static_cast<size_t>(tok) * D;
      } else if (pos < n0) {
        row = c.hot + (((static_cast<size_t>(b) * H + h) * T + (pos % T)) * 2 + kv) * D;
      } else {
        const _Float16* src = kv ? p.v_new : p.k_new;
        row = src + ((static_cast<size_t>(b) * p.max_n_new + (pos - n0)) * H + h) * D;
      }
    }
    x[v] = row ? *reinterpret_cast<const u32x4_t*>(row + col) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const int phys = __builtin_amdgcn_readfirstlane(ph_lane);
  const bool write = phys >= 0 && phys < c.num_phys;  // (workgroup-uniform; out-of-range ids are skipped)

  // ---- m = max |x| over the tile (exact: every candidate is an fp16 value)
  float m = 0.f;
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(half_lo(x[v][i])), fabsf(half_hi(x[v][i]))));
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
  // ---- s = fl32(m / L) (IEEE fp32 division), codes = clamp(rint(fl32(x / s)), -L, L)
  const float s = tile_scale<BITS>(m);
  float err;
  if (kv) {
    err = stage_cols<D, BITS, NV>(stage, x, s, tg, cg * 8, c.quant_err != nullptr);
  } else {
    err = stage_row<D, BITS, CPT, NV>(stage, x, s, 0, t, part * CPT, c.quant_err != nullptr);
  }
  const float tile_err = c.quant_err ? block_max(err, rerr) : 0.f;  // (also the stage barrier)
  __syncthreads();
  // ---- write the tile in its streaming layout
  if (write) {
    write_tile<D, BITS>(c.cold + tile_offset(phys, h, kv, H, TB), stage, kv, tid);
    if (tid == 0) c.scales[(static_cast<size_t>(phys) * H + h) * 2 + kv] = s;
    if (tid == 0 && c.quant_err) c.quant_err[(static_cast<size_t>(phys) * H + h) * 2 + kv] = tile_err;
    if (h == 0 && kv == 0 && tid == 0) {
      hdr->n_valid = valid;
      hdr->logical_block = j;
      hdr->flags = 0u;
    }
  }
}

// One workgroup per (sequence, kv-head): the tail shadow of the new partial block, then the hot ring.
// Each copy moves 16-byte vectors, item = (row, K|V, vector), kRingBatch per thread at a time: a
// round's loads are all issued before its stores (a store between them would make every load wait).
constexpr int kRingBatch = 8;

struct RingCopy {
  const _Float16* hot;     // this (sequence, kv-head)'s ring: [T][2][D]
  const _Float16* k_new;   // this (sequence, kv-head)'s first new token row (stride H*D per token)
  const _Float16* v_new;
  int n0, T, D, HD;
};

// Source of vector v of row (pos, kv): the ring slot (pos < n0) or the new token.
__device__ __forceinline__ const u32x4_t* ring_src(const RingCopy& r, int pos, int kv, int v) {
  const _Float16* row = pos < r.n0 ? r.hot + ((pos % r.T) * 2 + kv) * r.D
                                   : (kv ? r.v_new : r.k_new) + static_cast<size_t>(pos - r.n0) * r.HD;
  return reinterpret_cast<const u32x4_t*>(row) + v;
}

template <int D>
__global__ __launch_bounds__(kThreads) void append_ring_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int VPR = D / 8;            // 16-byte vectors per (token, head, K|V) row
  const CacheView& c = p.c;
  const int H = c.H, T = c.T;
  const int h = blockIdx.x % H;
  const int bl = blockIdx.x / H;
  if (bl >= p.n_seq) return;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  if (nn <= 0) return;
  const int n0 = p.n0[bl];  // the host mirror: this launch never reads seq_len, which it publishes
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t new0 = (static_cast<size_t>(b) * p.max_n_new * H + h) * D;
  const RingCopy r{c.hot + bh * T * 2 * D, p.k_new + new0, p.v_new + new0, n0, T, D, H * D};
  const int tid = threadIdx.x;

  // (1) FP16 shadow of the new partial last block (rows already there stay)
  const int jf = cold1 / S;
  if ((cold1 % S) != 0 && jf < c.max_blocks) {
    const int lo = max(jf * S, cold0);
    const int items = (cold1 - lo) * 2 * VPR;
    _Float16* tail = c.tail + bh * 2 * S * D;
    for (int base = 0; base < items; base += kRingBatch * kThreads) {
      u32x4_t buf[kRingBatch];
#pragma unroll
      for (int k = 0; k < kRingBatch; ++k) {
        const int it = min(base + k * kThreads + tid, items - 1);  // (clamped: every load is in range)
        buf[k] = *ring_src(r, lo + it / (2 * VPR), (it / VPR) % 2, it % VPR);
      }
#pragma unroll
      for (int k = 0; k < kRingBatch; ++k) {
        const int it = base + k * kThreads + tid;
        const int pos = lo + it / (2 * VPR), kv = (it / VPR) % 2;
        if (it < items) reinterpret_cast<u32x4_t*>(tail + (kv * S + (pos - jf * S)) * D)[it % VPR] = buf[k];
      }
    }
  }
  __syncthreads();  // ring slots read above are overwritten below
  // (2) new tokens that remain hot go to ring slot pos mod T
  {
    const int lo = max(n0, n1 - T);
    const int items = (n1 - lo) * 2 * VPR;
    _Float16* ring = c.hot + bh * T * 2 * D;
    for (int base = 0; base < items; base += kRingBatch * kThreads) {
      u32x4_t buf[kRingBatch];
#pragma unroll
      for (int k = 0; k < kRingBatch; ++k) {
        const int it = min(base + k * kThreads + tid, items - 1);  // (clamped: every load is in range)
        buf[k] = *ring_src(r, lo + it / (2 * VPR), (it / VPR) % 2, it % VPR);
      }
#pragma unroll
      for (int k = 0; k < kRingBatch; ++k) {
        const int it = base + k * kThreads + tid;
        const int pos = lo + it / (2 * VPR), kv = (it / VPR) % 2;
        if (it < items) reinterpret_cast<u32x4_t*>(ring + ((pos % T) * 2 + kv) * D)[it % VPR] = buf[k];
      }
    }
  }
  // the new length, once per sequence (no workgroup of this launch reads it)
  if (h == 0 && tid == 0) c.seq_len[b] = n1;
}

// Single-pass append, one workgroup per (sequence, kv-head), for appends that
// touch at most two cold blocks per sequence (a decode step touches one).
// Everything one kv-head of one sequence owns (its touched tiles, tail shadow
// rows and hot-ring slots) is handled by one workgroup, so no second launch is
// needed; the cached length comes from the host mirror (kernel argument), so
// no workgroup reads seq_len while another publishes it.
//
// One round of loads: every row the append needs (the spilled or new FP16 rows
// of the touched blocks, the old rows of a partial block from the tail
// shadow, the new tokens that stay hot) and the block headers are requested
// together at the start; nothing else is read.  In particular the old scale of
// a partial block is not loaded: its rows are the block's only rows, and
// s = fl32(m / 127) is monotonic and injective on fp16 maxima, so the stored
// scale is always fl32(m_old / 127) with m_old = max|x| over the tail-shadow
// rows.  When the new rows satisfy m_new <= m_old the block's maximum and scale
// are unchanged and only the new rows are coded (the old ones keep their
// codes); otherwise the whole block is re-quantised from its FP16 rows.  Both
// paths give the codes a full re-quantisation gives.
// 4-bit and fp16 tiles always re-write the whole touched block (a 4-bit row shares its V bytes
// with the neighbouring row, and an fp16 row's values never change).
template <int D, int BITS>
__global__ __launch_bounds__(kThreads) void append_step_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int TPT = kThreads / S;     // threads per token row
  constexpr int CPT = D / TPT;          // channels per thread
  constexpr int NV = CPT / 8;           // 16-byte vectors per thread and row
  constexpr int VPR = D / 8;            // 16-byte vectors per fp16 row
  constexpr int RING_V = 4;             // ring vectors per thread held in registers
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  __shared__ __align__(16) int8_t stage[TileStage<D, BITS>::BYTES];
  __shared__ float red[6][kWaves];
  __shared__ float rerr[kWaves];

  // grid (kv-head, sequence of this launch): no index depends on a kernel argument, so every
  // argument the kernel uses is read in one round of scalar loads, before any branch
  const int h = blockIdx.x;
  const int bl = blockIdx.y;
  const CacheView c = p.c;
  const _Float16* const k_new = p.k_new;
  const _Float16* const v_new = p.v_new;
  const int max_n_new = p.max_n_new;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  const int n0 = p.n0[bl];
  const int n_seq = p.n_seq;
  // consume every argument here: their scalar loads are issued together and waited for once,
  // instead of being sunk one by one behind the branches below
  asm volatile("" ::"s"(c.hot), "s"(c.tail), "s"(c.cold), "s"(c.scales), "s"(c.headers), "s"(c.seq_len),
               "s"(k_new), "s"(v_new), "s"(max_n_new), "s"(b), "s"(nn), "s"(n0), "s"(n_seq), "s"(c.H), "s"(c.T),
               "s"(c.max_blocks), "s"(c.num_phys));
  if (bl >= n_seq || nn <= 0) return;
  const int H = c.H, T = c.T;
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  const int tid = threadIdx.x;
  const int t = tid / TPT, part = tid % TPT;
  const size_t bh = static_cast<size_t>(b) * H + h;

  auto row_ptr = [&](int pos, int kv) -> const _Float16* {
    if (pos < n0) return c.hot + ((bh * T + (pos % T)) * 2 + kv) * D;
    return (kv ? v_new : k_new) + ((static_cast<size_t>(b) * max_n_new + (pos - n0)) * H + h) * D;
  };
  // row slices are ext-vector values (u32x4_t), never structs: selects between them stay in registers
  auto load_slice = [&](const _Float16* row, u32x4_t (&x)[NV]) {
    const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(row + part * CPT);
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] = r4[v];
  };
  auto zero_slice = [&](u32x4_t (&x)[NV]) {
#pragma unroll
    for (int v = 0; v < NV; ++v) x[v] = u32x4_t{0u, 0u, 0u, 0u};
  };
  auto slice_max = [&](const u32x4_t (&x)[NV]) -> float { return slice_absmax<NV>(x); };
  // codes of one row slice with scale s (as the IEEE division gives them, round half to even, clamp)
  auto code_slice = [&](const u32x4_t (&x)[NV], float s, uint32_t (&q)[CPT / 4]) {
    const float rs = quant_recip(s);
#pragma unroll
    for (int i = 0; i < CPT / 4; ++i) {
      uint32_t cb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = 4 * i + k;
        const uint32_t wd = x[e / 8][(e % 8) / 2];
        cb[k] = static_cast<uint32_t>(static_cast<int>(quant_code<127>((e & 1) ? half_hi(wd) : half_lo(wd), s, rs)));
      }
      q[i] = pack_low_bytes(cb[0], cb[1], cb[2], cb[3]);
    }
  };

  // ---- the touched blocks (at most two)
  const int j0 = cold0 / S;
  const int jl = cold1 > cold0 ? (cold1 - 1) / S : j0 - 1;  // last touched block
  const int nblk = jl >= j0 ? min(jl - j0 + 1, 2) : 0;
  const int v_old = cold0 - j0 * S;                         // coded rows of block j0 (tail shadow)
  int phys[2] = {-1, -1};  // raw header values; checked against [0, num_phys) where used
  u32x4_t xo[2][NV];      // old rows of block j0, K and V
  u32x4_t xn[2][2][NV];   // new rows of the touched blocks, [block][K|V]
  // the block index q is a compile-time constant in every use (keeps the row slices in registers)
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  auto load_block = [&](auto qc) {
    constexpr int q = decltype(qc)::value;
    const int j = j0 + q;
    const int lo = q == 0 ? v_old : 0;
    const int hi = q < nblk ? min(S, cold1 - j * S) : 0;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      if (t >= lo && t < hi) load_slice(row_ptr(j * S + t, kv), xn[q][kv]);
      else zero_slice(xn[q][kv]);
    }
  };
  load_block(Q0{});
  load_block(Q1{});
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    if (nblk > 0 && t < v_old) load_slice(c.tail + ((bh * 2 + kv) * S + t) * D, xo[kv]);
    else zero_slice(xo[kv]);
  }
  // the new tokens that stay hot (ring slots pos mod T), held in registers until the spilled
  // slots they replace have been read
  const int rlo = max(n0, n1 - T);
  const int ritems = (n1 - rlo) * 2 * VPR;
  u32x4_t rv[RING_V];
#pragma unroll
  for (int k = 0; k < RING_V; ++k) {
    // unconditional load from a clamped (valid) item: no divergent branch around it; only items
    // below ritems are stored (ritems >= 2 * VPR since nn >= 1)
    const int it = min(tid + k * kThreads, ritems - 1);
    const int v = it % VPR, kv = (it / VPR) % 2, pos = rlo + it / (2 * VPR);
    rv[k] = reinterpret_cast<const u32x4_t*>(row_ptr(pos, kv))[v];
  }
  // headers last: none of the row loads above waits for them
#pragma unroll
  for (int q = 0; q < 2; ++q)
    if (q < nblk && j0 + q < c.max_blocks) phys[q] = c.headers[static_cast<size_t>(b) * c.max_blocks + j0 + q].phys_block;

  // ---- block maxima (one reduction round for all six values)
  float mx[6] = {slice_max(xo[0]), slice_max(xo[1]), slice_max(xn[0][0]), slice_max(xn[0][1]),
                 slice_max(xn[1][0]), slice_max(xn[1][1])};
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    mx[i] = wave_max_dpp(mx[i]);  // DPP + readlane: no LDS round trips
    if ((tid & 63) == 0) red[i][tid >> 6] = mx[i];
  }
  __syncthreads();  // also: every load above has completed, so spilled slots may be overwritten
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    float r = red[i][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = fmaxf(r, red[i][w]);
    mx[i] = r;
  }

  // ---- codes of the touched blocks
  auto code_block = [&](auto qc) {
    constexpr int q = decltype(qc)::value;
    if (q >= nblk) return;
    const int j = j0 + q;
    const int vo = q == 0 ? v_old : 0;
    const int vn = min(S, cold1 - j * S);
    const bool is_new = t >= vo && t < vn;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {  // unrolled: the slices stay in registers
      const float m_old = q == 0 ? mx[kv] : 0.f;
      const float m_new = mx[2 + 2 * q + kv];
      if (phys[q] < 0 || phys[q] >= c.num_phys) continue;
      int8_t* tile = c.cold + tile_offset(phys[q], h, kv, H, TB);
      if (BITS == 8 && vo > 0 && m_new <= m_old) {
        // ---- maximum unchanged: code only the new rows, in place (the debug error statistic
        // covers every row: the old rows' codes are recomputed for it)
        if (c.quant_err) {
          const float so = m_old / 127.0f;
          const float e = t < vo ? slice_err8(xo[kv], so) : (is_new ? slice_err8(xn[q][kv], so) : 0.f);
          const float te = block_max(e, rerr);
          if (tid == 0) c.quant_err[(static_cast<size_t>(phys[q]) * H + h) * 2 + kv] = te;
          __syncthreads();  // rerr is reused
        }
        if (is_new) {
          const float so = m_old / 127.0f;
          uint32_t qw[CPT / 4];
          code_slice(xn[q][kv], so, qw);
          if (kv == 0) {
#pragma unroll
            for (int ch = 0; ch < CPT / 16; ++ch) {
              const int dc = (part * CPT) / 16 + ch;
              reinterpret_cast<uint4*>(tile)[dc * S + t] =  // stored offset binary
                  make_uint4(qw[4 * ch] ^ kCodeOffsetWord, qw[4 * ch + 1] ^ kCodeOffsetWord,
                             qw[4 * ch + 2] ^ kCodeOffsetWord, qw[4 * ch + 3] ^ kCodeOffsetWord);
            }
          } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
              tile[((t / 16) * D + part * CPT + i) * 16 + (t % 16)] =
                  static_cast<int8_t>((qw[i / 4] >> (8 * (i % 4))) ^ 0x80u);
          }
        }
        continue;
      }
      // ---- (re-)quantise the whole block: old rows from the tail shadow, new rows as loaded
      const float s = tile_scale<BITS>(fmaxf(m_old, m_new));
      u32x4_t xs[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) xs[v] = t < vo ? xo[kv][v] : xn[q][kv][v];  // element-wise: no indexed arrays
      const float err = stage_row<D, BITS, CPT, NV>(stage, xs, s, kv, t, part * CPT, c.quant_err != nullptr);
      const float tile_err = c.quant_err ? block_max(err, rerr) : 0.f;
      __syncthreads();
      write_tile<D, BITS>(tile, stage, kv, tid);
      if (tid == 0) c.scales[(static_cast<size_t>(phys[q]) * H + h) * 2 + kv] = s;
      if (tid == 0 && c.quant_err) c.quant_err[(static_cast<size_t>(phys[q]) * H + h) * 2 + kv] = tile_err;
      __syncthreads();  // stage is reused
    }
    if (h == 0 && tid == 0 && j < c.max_blocks) {
      hkv_block_header* hdr = c.headers + static_cast<size_t>(b) * c.max_blocks + j;
      hdr->n_valid = vn;
      hdr->logical_block = j;
      hdr->flags = 0u;
    }
  };
  code_block(Q0{});
  code_block(Q1{});

  // ---- FP16 shadow of the new partial last block: its new rows, from registers
  if ((cold1 % S) != 0 && nblk > 0) {
    const int q = jl - j0;  // the partial block is the last touched one
    const int vo = q == 0 ? v_old : 0;
    const int vn = cold1 - jl * S;
    if (t >= vo && t < vn) {
#pragma unroll
      for (int kv = 0; kv < 2; ++kv) {
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(c.tail + ((bh * 2 + kv) * S + t) * D + part * CPT);
#pragma unroll
        for (int v = 0; v < NV; ++v) dst[v] = q == 0 ? xn[0][kv][v] : xn[1][kv][v];
      }
    }
  }
  // ---- new tokens that stay hot: ring slot pos mod T (every read of the slots they replace
  // happened before the barrier above)
#pragma unroll
  for (int k = 0; k < RING_V; ++k) {
    const int it = tid + k * kThreads;
    if (it < ritems) {
      const int v = it % VPR, kv = (it / VPR) % 2, pos = rlo + it / (2 * VPR);
      reinterpret_cast<u32x4_t*>(c.hot + ((bh * T + (pos % T)) * 2 + kv) * D)[v] = rv[k];
    }
  }
  for (int it = tid + RING_V * kThreads; it < ritems; it += kThreads) {  // hot zones larger than the registers
    const int v = it % VPR, kv = (it / VPR) % 2, pos = rlo + it / (2 * VPR);
    reinterpret_cast<uint4*>(c.hot + ((bh * T + (pos % T)) * 2 + kv) * D)[v] =
        reinterpret_cast<const uint4*>(row_ptr(pos, kv))[v];
  }
  if (h == 0 && tid == 0) c.seq_len[b] = n1;
}

template <typename K>
hipError_t launch1(K kernel, int grid, const AppendParams& p, const LaunchCtx& ctx) {
  if (grid <= 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <typename K>
hipError_t launch_grid(K kernel, dim3 grid, const AppendParams& p, const LaunchCtx& ctx) {
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_append_db(const AppendParams& p, const LaunchCtx& quant_ctx, const LaunchCtx& ring_ctx) {
  if (p.single_pass) return launch_grid(append_step_kernel<D, BITS>, dim3(p.c.H, p.n_seq), p, quant_ctx);
  const int qgrid = p.touched_max > 0 ? p.n_seq * p.touched_max * p.c.H * 2 : 0;
  const hipError_t e = launch1(append_quant_kernel<D, BITS>, qgrid, p, quant_ctx);
  return e == hipSuccess ? launch1(append_ring_kernel<D>, p.n_seq * p.c.H, p, ring_ctx) : e;
}

template <int D>
hipError_t launch_append_d(const AppendParams& p, const LaunchCtx& quant_ctx, const LaunchCtx& ring_ctx) {
  switch (p.c.bits) {
    case 8: return launch_append_db<D, 8>(p, quant_ctx, ring_ctx);
    case 4: return launch_append_db<D, 4>(p, quant_ctx, ring_ctx);
    case 0: return launch_append_db<D, 0>(p, quant_ctx, ring_ctx);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

using namespace detail;

// Single-pass appends (at most two touched blocks per sequence): grid (kv-head, sequence).
// Otherwise the quantise launch (sequence, touched block, kv-head) and the ring/tail launch.
hipError_t launch_append(const AppendParams& p, const LaunchCtx& quant_ctx, const LaunchCtx& ring_ctx) {
  return p.c.D == 128 ? launch_append_d<128>(p, quant_ctx, ring_ctx) : launch_append_d<64>(p, quant_ctx, ring_ctx);
}

}  // namespace hkv
