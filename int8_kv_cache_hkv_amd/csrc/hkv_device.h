// Device helpers shared by the libhkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv_internal.h"

namespace hkv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Make LDS written by some lanes of this wave visible to the other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float exp2_approx(float x) { return __builtin_amdgcn_exp2f(x); }

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

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Streaming 16-byte load of cold-tile data that is read once per call: the
// non-temporal hint keeps it from displacing reused lines in the caches
// (measured on MI355X: the decode access pattern reads 6.8 TB/s with it, 6.1
// without).
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// An index the compiler must treat as per-lane: a load through it stays a
// vector-register value instead of being turned into a scalar right after the
// load (which would make the wave wait for it there).  Used for uniform values
// that are needed only much later.
__device__ __forceinline__ size_t opaque_index(size_t i) {
  asm volatile("" : "+v"(i));
  return i;
}

// Fourth descriptor word of a raw buffer resource on gfx9-family GPUs (32-bit
// data format, no swizzle).
constexpr int kBufferDword3 = 0x00020000;

// Raw buffer resource over `bytes` bytes at `base` (bytes = 0: every load
// returns 0 without a memory access, so a load can be issued unconditionally).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufferDword3);
}

// Streaming 16-byte buffer load (non-temporal, like load_stream) at byte
// offset `off` of the resource.
__device__ __forceinline__ uint4 load_stream_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  // bit_cast, not a conversion: an implicit conversion from the builtin's vector type may splat
  const u32x4_t v = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2 /* nt */));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Largest |x| over the fp16 values of a row slice (finite values, as the cache holds): for
// non-negative fp16 values the order of the bit patterns as unsigned integers is the numeric order, so
// the largest magnitude is the packed unsigned 16-bit maximum of the patterns with the sign bit
// cleared, two values per operation.
template <int NV>
__device__ __forceinline__ float slice_absmax(const u32x4_t (&x)[NV]) {
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  u16x2_t m = {0, 0};
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, x[v][i] & 0x7fff7fffu));
  return half_lo(m.x > m.y ? m.x : m.y);
}

// Reciprocal of a block scale for the coding helpers below: fl32(1 / s), the correctly rounded IEEE
// division (once per block), or 0 for s = 0 (every value of such a block is 0, and so is its code).
__device__ __forceinline__ float quant_recip(float s) { return s > 0.f ? 1.f / s : 0.f; }

// The quotient fl32(x / s) without a division per element, r = quant_recip(s).  y = fl32(x r) is
// within two ulps of x / s; the residual x - y s is exact in one fma, and the correction step
// y + (x - y s) r, rounded once, is the correctly rounded quotient (Markstein's theorem for round to
// nearest, given the correctly rounded reciprocal).  Checked exhaustively on the host against the
// division for every fp16 x with |x| <= m and every fp16 block maximum m > 0 with s = fl32(m / L),
// L = 127 and L = 7 (10^9 pairs each): no difference, and |rint(x / s)| <= L throughout.
__device__ __forceinline__ float quant_quotient(float x, float s, float r) {
  const float y = x * r;
  return __builtin_fmaf(__builtin_fmaf(-y, s, x), r, y);
}

// Code of x under scale s >= 0 with largest magnitude LIMIT (127 for 8-bit, 7 for 4-bit tiles):
// clamp(rint(fl32(x / s)), -LIMIT, LIMIT), round half to even, exactly what the IEEE fp32 division
// followed by rint gives.  r = quant_recip(s).
template <int LIMIT>
__device__ __forceinline__ float quant_code(float x, float s, float r) {
  const float k = __builtin_rintf(quant_quotient(x, s, r));
  return fminf(static_cast<float>(LIMIT), fmaxf(-static_cast<float>(LIMIT), k));
}

// Code in its byte form: for |q| < 2^22 the sum q + 1.5 * 2^23 rounds q to an integer (half to even,
// as rint does) and holds it in its low mantissa bits, so the low byte of the sum's bits is the code
// in two's complement.  For quotients of values inside their block's maximum (|q| < LIMIT + 1/2).
__device__ __forceinline__ uint32_t code_bits(float q) { return __builtin_bit_cast(uint32_t, q + 0x1.8p23f); }

// The low bytes of a, b, c, d packed into one word, a in the lowest byte.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

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

// Byte offset of the (phys, head, K|V) tile inside the cold pool (tile_bytes per tile).
__device__ __forceinline__ size_t tile_offset(int phys, int h, int kv, int H, int tile_bytes) {
  return ((static_cast<size_t>(phys) * H + h) * 2 + kv) * static_cast<size_t>(tile_bytes);
}

// A wave's walk over its dense units: runs of CU = units_per_split units start
// at split * CU and repeat every nsplit * CU; inside a run the wave takes every
// 4th unit, CU / 4 of them.  Unit k of the walk (k = 0, 1, ...):
__device__ __forceinline__ int walk_unit(int k, int split, int nsplit, int CU, int w) {
  const int KR = CU / kWaves;
  const int run = k / KR;
  return (split + run * nsplit) * CU + w + kWaves * (k - run * KR);
}

// Physical blocks of walk units kb .. kb + 63, one per lane (-1 past the header
// table or for an out-of-range id): one coalesced load serves 64 units, and
// the walk reads them with readlane, so no header load waits inside the loop.
__device__ __forceinline__ int header_batch(const CacheView& c, int b, int kb, int split, int nsplit, int CU, int w,
                                            int lane) {
  asm volatile("" : "+s"(CU));  // keeps the division by CU / 4 here (rarely executed), not hoisted and kept live
  const int j = walk_unit(kb + lane, split, nsplit, CU, w);
  const __amdgpu_buffer_rsrc_t rh =
      make_rsrc(c.headers + static_cast<size_t>(b) * c.max_blocks, static_cast<uint32_t>(c.max_blocks) * 16u);
  const bool in_table = j < c.max_blocks;
  const int ph = __builtin_amdgcn_raw_buffer_load_b32(rh, in_table ? j * 16 : -1, 0, 0);  // phys_block at offset 0
  return (in_table && ph >= 0 && ph < c.num_phys) ? ph : -1;
}

// Physical block of logical block j of sequence b (-1 past the table or for
// an out-of-range id).  The offset is kept per lane so the wave does not wait
// for the load where it is issued.
__device__ __forceinline__ int header_load(const CacheView& c, int b, int j) {
  const __amdgpu_buffer_rsrc_t rh =
      make_rsrc(c.headers + static_cast<size_t>(b) * c.max_blocks, static_cast<uint32_t>(c.max_blocks) * 16u);
  const bool in_table = j < c.max_blocks;
  const int o = static_cast<int>(opaque_index(static_cast<uint32_t>(in_table ? j * 16 : -1)));
  const int ph = __builtin_amdgcn_raw_buffer_load_b32(rh, o, 0, 0);  // phys_block at offset 0
  return in_table ? ph : -1;
}
__device__ __forceinline__ int header_phys(const CacheView& c, int hv) {
  const int ph = __builtin_amdgcn_readfirstlane(hv);
  return (ph >= 0 && ph < c.num_phys) ? ph : -1;
}

// One claim on the (sequence, kv-head) unit counter, issued by the whole wave
// without a branch: the buffer resource covers only the counter's 4 bytes and
// lane l addresses byte 4l, so the range check drops every lane but lane 0
// (an out-of-range buffer atomic touches no memory).  The result is read
// (readfirstlane) only when the claimed unit is needed; a branch around the
// atomic, or a uniform address (combined by the compiler, which reads the
// result at once), would make the wave wait for it where it is issued.
__device__ __forceinline__ unsigned claim_issue(unsigned* work, int lane) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(work, 4u);
  return static_cast<unsigned>(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, r, lane * 4, 0, 0));
}

// Workgroup coordinates of a 3D grid (x = split, y = kv-head, z = sequence).
// Workgroups are dispatched round-robin over the 8 dies in linear order,
// and a workgroup dispatched earlier keeps a lead in memory bandwidth over the
// ones dispatched after it (measured: in a resident 131072-token launch the
// splits of the first sequence finished 47 us before those of the last).
// Orders (each a bijection of the grid):
//  * kOrderPlain: linear order; short splits (latency-bound steps), where it
//    measured fastest;
//  * kOrderSplitMajor: the linear order runs over (sequence, kv-head) first,
//    so every (sequence, kv-head) gets early and late workgroups alike, and
//    round k (split k) is rotated by k pairs, so its workgroups also visit
//    every die (the dies' bandwidths differ too: up to 25 % in one measured
//    launch); with dynamic unit claims the fast workgroups of a (sequence,
//    kv-head) take the larger share and all of them end together.
struct WgCoord {
  int x, y, z;
};
__device__ __forceinline__ WgCoord wg_coord(int order) {
  const int X = gridDim.x, Y = gridDim.y;
  if (order == kOrderPlain)
    return {static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z)};
  const int N = X * Y * static_cast<int>(gridDim.z);
  const int lin = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
  const int P = N / X;  // kOrderSplitMajor; (sequence, kv-head) pairs
  const int k = lin / P;
  const int pair = (lin - k * P + k) % P;
  return {k, pair % Y, pair / Y};
}

// kOrderTable (batch plans, whose grid runs in several rounds of the resident
// slots): a grid of H x groups workgroups, group g being the H kv-heads of one
// (sequence, part) of the host-built table `order` of (sequence << 7 | part)
// entries (only the parts that sequence takes part with).  Returns x = part,
// y = kv-head, z = sequence as for the other orders.
__device__ __forceinline__ WgCoord wg_coord_table(const uint16_t* order) {
  // grid (H, groups): the H kv-heads of group blockIdx.y are consecutive in dispatch order
  const int e = order[blockIdx.y];
  return {e & 127, static_cast<int>(blockIdx.x), e >> 7};
}

// ---------------------------------------------------------------- MFMA / DPP helpers
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// One step of a wave maximum: x = max(x, x of the lane the DPP control names), a single v_max_f32
// with a DPP source (through a DPP move, fmaxf costs the move, a NaN-canonicalising max and the
// max).  The s_nop gives the two wait states a DPP read needs after a VALU write of its source.
// Rows outside the row mask keep x.  For the values maximised here (never a signalling NaN) this is
// fmaxf.
#define HKV_MAX_DPP_STEP(name, ctrl)                                                     \
  __device__ __forceinline__ float name(float x) {                                       \
    asm("s_nop 1\n\tv_max_f32_dpp %0, %0, %0 " ctrl : "+v"(x));                         \
    return x;                                                                            \
  }
HKV_MAX_DPP_STEP(max_dpp_quad_swap1, "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf")
HKV_MAX_DPP_STEP(max_dpp_quad_swap2, "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf")
HKV_MAX_DPP_STEP(max_dpp_half_mirror, "row_half_mirror row_mask:0xf bank_mask:0xf")
HKV_MAX_DPP_STEP(max_dpp_mirror, "row_mirror row_mask:0xf bank_mask:0xf")
HKV_MAX_DPP_STEP(max_dpp_bcast15, "row_bcast:15 row_mask:0xa bank_mask:0xf")
HKV_MAX_DPP_STEP(max_dpp_bcast31, "row_bcast:31 row_mask:0xc bank_mask:0xf")
#undef HKV_MAX_DPP_STEP

// Max over the 64 lanes, wave-uniform result: inside rows of 16 lanes by quad swaps and row
// mirrors, then row 1 takes row 0's and row 3 row 2's (row_bcast:15), row 3 takes row 1's
// (row_bcast:31), and lane 63 holds the maximum.
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = max_dpp_quad_swap1(x);
  x = max_dpp_quad_swap2(x);
  x = max_dpp_half_mirror(x);
  x = max_dpp_mirror(x);
  x = max_dpp_bcast15(x);
  x = max_dpp_bcast31(x);
  return readlane_f(x, 63);
}

// Sum over the 64 lanes, wave-uniform result: DPP inside rows of 16 lanes, then the four row
// sums read as scalars and added in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

// 8-bit codes are stored offset binary: byte = code + 128 (code -127..127 is stored 1..255,
// code 0 as 0x80), so a byte placed under the fp16 exponent of 1024 is the exact value
// code + 1152 with no work on the byte itself.
constexpr uint32_t kCodeOffsetWord = 0x80808080u;  // the offset of four code bytes (an exclusive or)

// Four stored 8-bit codes (one word) to four exact fp16 values: each byte under the fp16
// exponent of 1024 (0x64xx = 1024 + byte = code + 1152), minus 1152.  Every step is exact.
__device__ __forceinline__ half4_t codes_to_half4(uint32_t u) {
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t off = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  const half2_t a = __builtin_bit_cast(half2_t, lo) - off;
  const half2_t b = __builtin_bit_cast(half2_t, hi) - off;
  return half4_t{a.x, a.y, b.x, b.y};
}

// Four stored 8-bit codes (one word) to the four exact fp16 values code + 1152: the same byte
// placement as codes_to_half4 without the final subtraction.  Callers remove the 1152 offset from
// the finished dot products.
__device__ __forceinline__ half4_t codes_to_biased_half4(uint32_t u) {
  const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const half2_t a = __builtin_bit_cast(half2_t, lo);
  const half2_t b = __builtin_bit_cast(half2_t, hi);
  return half4_t{a.x, a.y, b.x, b.y};
}
constexpr float kCodeBias = 1152.0f;

// ---------------------------------------------------------------- cold-tile formats
// One cold tile holds the S = 64 tokens x D channels of one (block, kv-head, K|V) as 8-bit codes,
// 4-bit codes or fp16 values (quant_bits 8, 4, 0), in 16-byte chunks laid out so that one coalesced
// wave load gives every lane its MFMA operand:
//   K tile: chunk (kc, t) at byte (kc * S + t) * 16 holds channels [kc * E, kc * E + E) of token t;
//   V tile: chunk (vc, c) at byte (vc * D + c) * 16 holds tokens [vc * E, vc * E + E) of channel c;
// E = elements per chunk (16, 32 or 8).  Element e of a chunk is byte e (8-bit, offset binary), a
// nibble holding code + 8 (4-bit, offset binary, code 0 is 8; planar per word: see nib_byte), or
// bytes 2e, 2e + 1 (fp16).  An FP16 tile's scale is stored as 1.
template <int BITS>
struct Fmt {
  static_assert(BITS == 8 || BITS == 4 || BITS == 0, "8-bit, 4-bit or fp16 tiles");
  static constexpr int kElems = BITS == 8 ? 16 : (BITS == 4 ? 32 : 8);  // elements per 16-byte chunk
  static constexpr int kSteps = kElems / 4;                            // 4-element MFMA operands per chunk
  static constexpr int kLimit = BITS == 8 ? 127 : 7;                   // largest code magnitude
  // 8-bit QK operands are biased (no subtraction per element): code + kBias, removed from each logit.
  // The removal's fp32 rounding (relative to the offset sum) is multiplied by the block scale, which
  // is 127/7 times larger at 4 bits for the same maximum: 4-bit QK operands are the exact codes.
  static constexpr bool kBiasedQK = BITS == 8;
  static constexpr float kBias = BITS == 8 ? kCodeBias : 0.0f;
  template <int D>
  static constexpr int tile_bytes() { return BITS == 0 ? 64 * D * 2 : 64 * D * BITS / 8; }
};

// 4-bit chunks are planar per 32-bit word: word j holds elements 8j..8j+3 in the low nibbles of its
// bytes 0..3 and elements 8j+4..8j+7 in the high nibbles (offset binary, code + 8).  Byte and shift of
// element r of a chunk:
__device__ __forceinline__ int nib_byte(int r) { return (r >> 3) * 4 + (r & 3); }
__device__ __forceinline__ int nib_shift(int r) { return ((r >> 2) & 1) * 4; }

// MFMA operand `step` (4 consecutive elements) of a 16-byte chunk, as fp16 values: biased
// (code + kBias, the QK operand) or exact (the code itself, the PV operand).  fp16 tiles give the
// values themselves either way.
template <int BITS, bool BIASED>
__device__ __forceinline__ half4_t chunk_operand(const uint4& ck, int step) {
  if constexpr (BITS == 8) {
    return BIASED ? codes_to_biased_half4(word_of(ck, step)) : codes_to_half4(word_of(ck, step));
  } else if constexpr (BITS == 4) {
    // the step's four nibbles, one per byte (the low half of its word, or the high half), each
    // placed under the fp16 exponent of 1024 by one byte permute: 1024 + nibble, exact
    const uint32_t w = word_of(ck, step >> 1);
    const uint32_t n = ((step & 1) ? (w >> 4) : w) & 0x0F0F0F0Fu;
    half2_t a = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n, 0x04010400u));
    half2_t b = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, n, 0x04030402u));
    if (!BIASED) {
      const half2_t off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
      a = a - off;
      b = b - off;
    }
    return half4_t{a.x, a.y, b.x, b.y};
  } else {
    const uint2 v = step == 0 ? make_uint2(ck.x, ck.y) : make_uint2(ck.z, ck.w);
    return __builtin_bit_cast(half4_t, v);
  }
}

__device__ __forceinline__ float4_t mfma_qk(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, c, 0, 0, 0);
}

// 4-bit tiles: eight int8 codes (x0: elements 0..3, x1: 4..7) as one planar word of offset-binary
// nibbles (elements 0..3 low, 4..7 high).  (c & 15) ^ 8 = c + 8 for c in [-7, 7].
__device__ __forceinline__ uint32_t pack_nib8(uint32_t x0, uint32_t x1) {
  const uint32_t a = (x0 & 0x0F0F0F0Fu) ^ 0x08080808u;
  const uint32_t b = (x1 & 0x0F0F0F0Fu) ^ 0x08080808u;
  return a | (b << 4);
}

// A 16-byte tile chunk from 16 bytes of stage (8-bit codes or fp16 values), or from 32 code bytes
// packed into nibbles (4-bit).
template <int BITS>
__device__ __forceinline__ uint4 chunk_from_stage(const int8_t* src) {
  if constexpr (BITS == 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    const uint4 b = *reinterpret_cast<const uint4*>(src + 16);
    return make_uint4(pack_nib8(a.x, a.y), pack_nib8(a.z, a.w), pack_nib8(b.x, b.y), pack_nib8(b.z, b.w));
  } else if constexpr (BITS == 8) {  // signed stage codes to the stored offset-binary bytes
    const uint4 a = *reinterpret_cast<const uint4*>(src);
    return make_uint4(a.x ^ kCodeOffsetWord, a.y ^ kCodeOffsetWord, a.z ^ kCodeOffsetWord, a.w ^ kCodeOffsetWord);
  } else {
    return *reinterpret_cast<const uint4*>(src);
  }
}

}  // namespace hkv
