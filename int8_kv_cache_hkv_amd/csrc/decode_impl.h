// Split-K decode attention over the hybrid cache, and its log-sum-exp combine
// (gfx950, wave64, MFMA).
//
// out[b][hq] = softmax(q . K^T / sqrt(d)) . V over the FP16 hot zone and the
// dequantised INT8 cold blocks (Hybrid KV Cache page 2.1 and 4.2: hot part in
// full precision, cold blocks dequantised on read; here one joint softmax).
//
// Work decomposition.  For each (sequence, kv-head) the cold tokens are split
// into "units": unit j is cold block j (dense mode) or the j-th run of 16
// selected cold tokens (sparse mode, KV Cache reuse page 2: only the selected
// tokens are loaded).  A workgroup of 4 waves owns one split = a run of
// units_per_split units (round-robin over runs when a sequence has more units
// than the grid covers); each wave streams every 4th unit of the run and keeps
// an fp32 online softmax (m, l, acc) for the G query heads of the kv-head; the
// 4 waves are merged in LDS into one partial per split.  One more workgroup
// per (sequence, kv-head) attends the FP16 hot zone, and the last workgroup to
// finish merges all partials.
//
// Per unit of 64 tokens a wave does (all on v_mfma_f32_4x4x4f16):
//   QK  B operand = 4 channels of the lane's own token (lane = token), A
//       operand = 4 channels of query row lane%4 (from LDS), so lane t ends
//       with the logits of token t for 4 query heads.
//   PV  B operand = the value codes of 4 consecutive tokens at the lane's
//       channel (lane = channel), A operand = the weights of those tokens for
//       query row lane%4 (from LDS), so lane c accumulates out[g][c].
// Key codes enter the QK MFMAs as the exact fp16 values code + 1152 (a byte
// permute under the fp16 exponent of 1024; no subtraction), and 1152 * sum(q)
// is removed from each finished logit.  Value codes enter the PV MFMAs as the
// exact codes: an offset there would have to be cancelled from sums of size
// 1152 * s_V, which costs absolute accuracy when s_V is large (fp16-range
// values).  Weights are p = 2^(z - block max) in [0, 1], split into hi + lo
// fp16 halves (about 22 significant bits) and accumulated per block; the
// block's V scale and its online-softmax factor are applied once per block in
// fp32.
// Cold tiles are laid out so that one coalesced 16-byte load per lane lands
// exactly these operands: lane t gets 16 channels of token t from a K tile,
// lane c gets 16 tokens of channel c from a V tile.  Dense units are software
// pipelined: each 1 KiB chunk of the current K (V) tile is replaced by the same
// chunk of the next unit's tile as soon as its QK (PV) products are issued, so
// a wave always has about one unit's loads in flight.
//
// Cold tiles come in three formats (8-bit codes, 4-bit codes, fp16 values; see Fmt): every
// function that touches a tile takes the format as the template parameter BITS.  Each (head_dim,
// group, format) instance is compiled from decode_inst.hip into an object of its own.
#pragma once

#include <hip/hip_ext.h>

#include <cstring>
#include <type_traits>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr float kNegInf = -__builtin_inff();
constexpr int kModeDense = 0;   // cold blocks of the header table
constexpr int kModeGather = 1;  // selected tokens gathered from their blocks (sel_idx)
constexpr int kModeStore = 2;   // units of a compacted sparse store
constexpr int kHotChunk = 32;         // hot-zone slots staged through LDS at a time
constexpr int kMergeChunk = 16;       // partials whose loads are in flight together in the merge

template <int D, int G>
struct Cfg {
  static constexpr int NQ = (G + 3) / 4;   // groups of 4 query heads (MFMA rows)
  static constexpr int NG = 4 * NQ;        // query rows including zero padding
  static constexpr int NDL = D / 64;       // channel passes of 64 lanes
  static constexpr int QROW = D + 8;       // padded fp16 query row in LDS (spreads the 4 rows over banks)
  static constexpr int PROW = 16 * 8 + 8;  // fp16 weight row: 16 groups of {hi[4], lo[4]}, padded
};

template <int D, int G>
struct DecodeSmem {
  using C = Cfg<D, G>;
  alignas(16) _Float16 qh[C::NQ][4][C::QROW];        // query rows (fp16, exact), zero rows past G
  alignas(16) _Float16 pw[kWaves][C::NQ][4][C::PROW]; // per-wave weights of the current unit (hi/lo)
  float wm[kWaves][C::NG];
  float wl[kWaves][C::NG];
  float wz[kWaves][C::NG];                          // per-wave sums of w * logit (entropy statistic)
  alignas(16) float wacc[kWaves][C::NG][D];
};

template <int D, int G>
struct HotSmem {
  using C = Cfg<D, G>;
  alignas(16) _Float16 qh[C::NQ][4][C::QROW];          // query rows (fp16), zero rows past G
  float acc[G][D];
  float z[C::NG][kHotChunk];               // softmax weights of the current chunk (rows stay 0 past cnt)
  float m[C::NG], l[C::NG], zs[C::NG], alpha[C::NG];
  alignas(16) _Float16 kv[kHotChunk * (2 * D + 8)];     // staged [K|V] rows of the current chunk (padded)
};

// Per-block PV sums: one MFMA chain per (query quad, channel pass); the hi and lo
// weight halves accumulate into the same chain.
template <int D, int G>
struct BlockAcc {
  float4_t v[Cfg<D, G>::NQ][Cfg<D, G>::NDL];
};

template <int D, int G>
struct WaveState {
  using C = Cfg<D, G>;
  float m[C::NG];                          // running max of base-2 logits (wave-uniform)
  float l[C::NG];                          // lane-partial sum of softmax weights
  bool stats;                              // carry the entropy statistic (the cache view asks for it)
  float qb[C::NG];                         // bias * sum_k q[g][k] (wave-uniform; see Fmt::kBias)
  float4_t acc[C::NQ][C::NDL];             // out[4quad + r][64 pass + lane] (with the code offset)
};

// Lane-partial sums of weight * logit (entropy statistic) of wave w's row g: kept in the wave's own
// wacc rows, which the wave writes only after it has read them back (LDS operations of one wave stay
// in order), so the statistic costs no registers in the unit loop.
template <int D, int G>
__device__ __forceinline__ float& z_lane(DecodeSmem<D, G>& sm, int w, int g, int lane) {
  static_assert(D >= 64, "the per-lane sums of a wave fit its wacc rows");
  return (&sm.wacc[w][0][0])[g * 64 + lane];
}

template <int D, int G>
__device__ __forceinline__ half4_t q_operand(const DecodeSmem<D, G>& sm, int quad, int lane, int k0) {
  return *reinterpret_cast<const half4_t*>(&sm.qh[quad][lane & 3][k0]);
}

// Online-softmax update for one unit.  s[quad][r]: this lane's logit sums for
// query row 4quad + r with biased key codes; `scale` (per lane) turns
// s - qb into a base-2 logit; masked lanes give weight 0.  Per query row the
// block max mb is taken first, the weight is w = 2^(z - mb) * vw (vw <= 1 per
// lane, the lane's V scale relative to vcoef), stored to LDS as hi/lo fp16 for
// the PV MFMAs, and the row's fold factors are returned: alpha rescales the
// old accumulator, coef multiplies this block's PV sum.
template <int D, int G, bool PER_LANE_V>
__device__ __forceinline__ void softmax_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const float4_t (&s)[Cfg<D, G>::NQ],
                                             bool valid, float scale, float vw, float vcoef,
                                             float (&alpha)[Cfg<D, G>::NG], float (&coef)[Cfg<D, G>::NG], int w, int lane) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * quad + r;
      const float z = valid ? (s[quad][r] - st.qb[g]) * scale : kNegInf;
      const float mb = wave_max_dpp(z);
      const bool none = mb == kNegInf;  // every lane masked: state unchanged
      const float mn = fmaxf(st.m[g], mb);
      const float a = none ? 1.f : exp2_approx(st.m[g] - mn);
      const float be = none ? 0.f : exp2_approx(mb - mn);
      const float pp = none ? 0.f : exp2_approx(z - mb);
      const float wv = PER_LANE_V ? pp * vw : pp;
      const float cf = be * vcoef;
      st.l[g] = fmaf(st.l[g], a, be * pp);
      st.m[g] = mn;
      alpha[g] = a;
      coef[g] = cf;
      const _Float16 hi = static_cast<_Float16>(wv);
      const _Float16 lo = static_cast<_Float16>(wv - static_cast<float>(hi));
      _Float16* row = &sm.pw[w][quad][r][(lane >> 2) * 8 + (lane & 3)];
      row[0] = hi;
      row[4] = lo;
    }
  }
  // entropy statistic, outside the row loop so that it holds no registers there: the weight
  // 2^(z - m) of the new maximum m (equal to 2^(mb - m) 2^(z - mb) up to rounding)
  if (st.stats) {
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = 4 * quad + r;
        const float z = (s[quad][r] - st.qb[g]) * scale;
        float& zl = z_lane(sm, w, g, lane);
        zl = fmaf(zl, alpha[g], valid && st.m[g] != kNegInf ? exp2_approx(z - st.m[g]) * z : 0.f);
      }
    }
  }
  wave_lds_sync();
}

// The weights (hi and lo halves) of tokens t0 .. t0 + 3 for every query quad, from wave w's rows.
template <int D, int G>
__device__ __forceinline__ void pv_weights(const DecodeSmem<D, G>& sm, int t0, int w, int lane,
                                           half4_t (&ph)[Cfg<D, G>::NQ], half4_t (&pl)[Cfg<D, G>::NQ]) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) {
    const half4_t* pr = reinterpret_cast<const half4_t*>(&sm.pw[w][quad][lane & 3][(t0 >> 2) * 8]);
    ph[quad] = pr[0];
    pl[quad] = pr[1];
  }
}

// PV products of 4 tokens: both weight halves into the same chain.
template <int D, int G>
__device__ __forceinline__ void pv_mfma(BlockAcc<D, G>& blk, const half4_t (&ph)[Cfg<D, G>::NQ],
                                        const half4_t (&pl)[Cfg<D, G>::NQ], const half4_t (&bv)[Cfg<D, G>::NDL]) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) blk.v[quad][ps] = mfma_qk(ph[quad], bv[ps], blk.v[quad][ps]);
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) blk.v[quad][ps] = mfma_qk(pl[quad], bv[ps], blk.v[quad][ps]);
}

// PV products of four tokens t0..t0+3 into the block accumulators: bv[ps] is the exact value
// operand (the four tokens' values at channel 64 ps + lane).
template <int D, int G>
__device__ __forceinline__ void pv_step(BlockAcc<D, G>& blk, const DecodeSmem<D, G>& sm,
                                        const half4_t (&bv)[Cfg<D, G>::NDL], int t0, int w, int lane) {
  using C = Cfg<D, G>;
  half4_t ph[C::NQ], pl[C::NQ];
  pv_weights<D, G>(sm, t0, w, lane, ph, pl);
  pv_mfma<D, G>(blk, ph, pl, bv);
}

template <int D, int G>
__device__ __forceinline__ void zero_blk(BlockAcc<D, G>& blk) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) blk.v[quad][ps] = float4_t{0.f, 0.f, 0.f, 0.f};
}

// acc = acc * alpha + coef * block sum, per query row.
template <int D, int G>
__device__ __forceinline__ void fold_block(WaveState<D, G>& st, const BlockAcc<D, G>& blk,
                                           const float (&alpha)[Cfg<D, G>::NG], const float (&coef)[Cfg<D, G>::NG]) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int g = 4 * quad + r;
        st.acc[quad][ps][r] = fmaf(coef[g], blk.v[quad][ps][r], st.acc[quad][ps][r] * alpha[g]);
      }
}

// The query operands of K chunk ch (kSteps MFMA steps) for every query quad.
template <int D, int G, int BITS>
__device__ __forceinline__ void q_chunk(const DecodeSmem<D, G>& sm, int lane, int ch,
                                        half4_t (&q)[Fmt<BITS>::kSteps][Cfg<D, G>::NQ]) {
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
#pragma unroll
  for (int st = 0; st < F::kSteps; ++st)
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad) q[st][quad] = q_operand(sm, quad, lane, ch * F::kElems + st * 4);
}

// Logit sums of the lane's K row (D/E chunks of E elements, biased operands) for every query row.
// The query operands of the next chunk are read from LDS while this chunk's MFMAs run (a read
// issued right before its MFMA leaves the LDS latency exposed at one wave per SIMD).
template <int D, int G, int BITS>
__device__ __forceinline__ void qk_codes(const uint4 (&kr)[D / Fmt<BITS>::kElems], const DecodeSmem<D, G>& sm,
                                         int lane, float4_t (&s)[Cfg<D, G>::NQ]) {
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
  constexpr int NCH = D / F::kElems;
  asm volatile("" ::: "memory");  // re-read the query operand from LDS for every unit
  float4_t s2[C::NQ];  // second accumulator chain: halves the dependent MFMA chain
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] = s2[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
  half4_t qc[F::kSteps][C::NQ];
  q_chunk<D, G, BITS>(sm, lane, 0, qc);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    asm volatile("" ::: "memory");  // bound how far the query-operand LDS reads are hoisted
    half4_t qn[F::kSteps][C::NQ];
    if (ch + 1 < NCH) q_chunk<D, G, BITS>(sm, lane, ch + 1, qn);
#pragma unroll
    for (int st = 0; st < F::kSteps; ++st) {
      const half4_t b = chunk_operand<BITS, F::kBiasedQK>(kr[ch], st);
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) {
        if (st & 1) s2[quad] = mfma_qk(qc[st][quad], b, s2[quad]);
        else s[quad] = mfma_qk(qc[st][quad], b, s[quad]);
      }
    }
    if (ch + 1 < NCH) {
#pragma unroll
      for (int st = 0; st < F::kSteps; ++st)
#pragma unroll
        for (int quad = 0; quad < C::NQ; ++quad) qc[st][quad] = qn[st][quad];
    }
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] += s2[quad];
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- dense units
// QK of a dense unit with progressive refill: as soon as chunk ch of the K tile
// has been turned into MFMA operands, its registers receive chunk ch of the
// next unit's K tile (rn; an empty descriptor when there is none), so the next
// tile is requested chunk by chunk while this one is consumed.
template <int D, int G, int BITS>
__device__ __forceinline__ void qk_codes_refill(uint4 (&kr)[D / Fmt<BITS>::kElems], const DecodeSmem<D, G>& sm,
                                                int lane, float4_t (&s)[Cfg<D, G>::NQ], __amdgpu_buffer_rsrc_t rn) {
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
  constexpr int S = kBlockSize;
  constexpr int NCH = D / F::kElems;
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
  asm volatile("" ::: "memory");
  float4_t s2[C::NQ];
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] = s2[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
  half4_t qc[F::kSteps][C::NQ];  // this chunk's query operands; the next chunk's are read meanwhile
  q_chunk<D, G, BITS>(sm, lane, 0, qc);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    asm volatile("" ::: "memory");
    half4_t qn[F::kSteps][C::NQ];
    if (ch + 1 < NCH) q_chunk<D, G, BITS>(sm, lane, ch + 1, qn);
#pragma unroll
    for (int st = 0; st < F::kSteps; ++st) {
      const half4_t b = chunk_operand<BITS, F::kBiasedQK>(kr[ch], st);
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) {
        if (st & 1) s2[quad] = mfma_qk(qc[st][quad], b, s2[quad]);
        else s[quad] = mfma_qk(qc[st][quad], b, s[quad]);
      }
    }
    kr[ch] = load_stream_buf(rn, lo + ch * S * 16);
    if (ch + 1 < NCH) {
#pragma unroll
      for (int st = 0; st < F::kSteps; ++st)
#pragma unroll
        for (int quad = 0; quad < C::NQ; ++quad) qc[st][quad] = qn[st][quad];
    }
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] += s2[quad];
  asm volatile("" ::: "memory");
}

// PV of a dense unit with progressive refill: once the last operand of a column
// chunk (E tokens of the lane's channel) has been used, its registers receive
// the same chunk of the next unit's V tile.
template <int D, int G, int BITS>
__device__ __forceinline__ void pv_dense_refill(BlockAcc<D, G>& blk, const DecodeSmem<D, G>& sm,
                                                uint4 (&vr)[Cfg<D, G>::NDL][64 / Fmt<BITS>::kElems], int w,
                                                int lane, __amdgpu_buffer_rsrc_t rn) {
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
  constexpr int S = kBlockSize;
  constexpr int E = F::kElems;
  constexpr int TB = F::template tile_bytes<D>();
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
  zero_blk<D, G>(blk);
  half4_t ph[C::NQ], pl[C::NQ];  // this step's weights; the next step's are read meanwhile
  pv_weights<D, G>(sm, 0, w, lane, ph, pl);
#pragma unroll
  for (int t0 = 0; t0 < S; t0 += 4) {
    asm volatile("" ::: "memory");
    half4_t nh[C::NQ], nl[C::NQ];
    if (t0 + 4 < S) pv_weights<D, G>(sm, t0 + 4, w, lane, nh, nl);
    half4_t bv[C::NDL];
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) bv[ps] = chunk_operand<BITS, false>(vr[ps][t0 / E], (t0 % E) / 4);
    pv_mfma<D, G>(blk, ph, pl, bv);
    if (t0 + 4 < S) {
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) {
        ph[quad] = nh[quad];
        pl[quad] = nl[quad];
      }
    }
    if (t0 % E == E - 4) {
#pragma unroll
      for (int ps = 0; ps < C::NDL; ++ps)
        vr[ps][t0 / E] = load_stream_buf(rn, lo + TB + ((t0 / E) * D + 64 * ps) * 16);
    }
  }
  asm volatile("" ::: "memory");
}

// The two scales (K, V) of a block; phys < 0 reads 0.  The offset is kept per
// lane so the wave does not wait for the load right after issuing it.
__device__ __forceinline__ float2 load_scales(__amdgpu_buffer_rsrc_t rs, int phys, int H, int h) {
  const int so = static_cast<int>(opaque_index(static_cast<uint32_t>((phys * H + h) * 8)));
  const int o = phys < 0 ? -8 : so;
  return make_float2(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0)),
                     __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 4, 0)));
}

// One dense unit's tiles in registers.
template <int D, int BITS>
struct Tiles {
  static constexpr int E = Fmt<BITS>::kElems;
  uint4 kr[D / E];         // lane t: chunk ch = elements E ch .. E ch + E - 1 of token t
  uint4 vr[D / 64][64 / E];  // lane c: [pass][vc] = tokens E vc .. E vc + E - 1 of channel 64 pass + lane
};

// Buffer resource over one block's K and V tiles of one kv-head (2 tile_bytes
// contiguous bytes, K first): the tile loads take a uniform descriptor plus a
// 32-bit lane offset, and the hardware range check returns 0 past the end.
// phys < 0 gives an empty descriptor: the loads return 0 and touch no memory.
template <int D, int BITS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const CacheView& c, int phys, int h) {
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  const bool ok = phys >= 0;
  const int8_t* base = c.cold + tile_offset(ok ? phys : 0, h, 0, c.H, TB);
  return make_rsrc(base, ok ? 2u * TB : 0u);
}

// Descriptor over the whole scales array [num_phys][H][2]: an out-of-range
// (phys, h) reads 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scales_rsrc(const CacheView& c) {
  return make_rsrc(c.scales, static_cast<uint32_t>(c.num_phys) * c.H * 8u);
}

// Request the K tile (lane t: E elements of token t per chunk).
template <int D, int BITS>
__device__ __forceinline__ void issue_k(Tiles<D, BITS>& t, __amdgpu_buffer_rsrc_t r, int lane) {
  constexpr int S = kBlockSize;
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int ch = 0; ch < D / Fmt<BITS>::kElems; ++ch) t.kr[ch] = load_stream_buf(r, lo + ch * S * 16);
}

// Request the two scales (K, V) and the V tile (lane c: E tokens of channel c
// per load).  The scales travel with the V tile: they are requested after the
// previous unit's softmax has used the register pair.
template <int D, int BITS>
__device__ __forceinline__ void issue_v(Tiles<D, BITS>& t, float2& sc, __amdgpu_buffer_rsrc_t r,
                                        __amdgpu_buffer_rsrc_t rs, int phys, int H, int h, int lane) {
  constexpr int E = Fmt<BITS>::kElems;
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  // per-lane offset (kept out of scalar registers: no wait right after the load); phys < 0 reads 0
  const int so = static_cast<int>(opaque_index(static_cast<uint32_t>((phys * H + h) * 8)));
  // two 32-bit loads (the 64-bit buffer-load builtin can come out as a single dword load)
  const int o = phys < 0 ? -8 : so;
  sc = make_float2(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 0, 0)),
                   __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, o, 4, 0)));
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int ps = 0; ps < D / 64; ++ps)
#pragma unroll
    for (int vc = 0; vc < 64 / E; ++vc) t.vr[ps][vc] = load_stream_buf(r, lo + TB + (vc * D + 64 * ps) * 16);
}

// PV over a dense unit whose values are lane-resident: vr[pass][vc] holds
// tokens E vc .. E vc + E - 1 of channel 64 pass + lane.
template <int D, int G, int BITS>
__device__ __forceinline__ void pv_dense(BlockAcc<D, G>& blk, const DecodeSmem<D, G>& sm,
                                         const uint4 (&vr)[Cfg<D, G>::NDL][64 / Fmt<BITS>::kElems], int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int E = Fmt<BITS>::kElems;
  zero_blk<D, G>(blk);
#pragma unroll
  for (int t0 = 0; t0 < 64; t0 += 4) {
    asm volatile("" ::: "memory");  // read the weights 4 tokens at a time (bounds live VGPRs)
    half4_t bv[C::NDL];
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) bv[ps] = chunk_operand<BITS, false>(vr[ps][t0 / E], (t0 % E) / 4);
    pv_step<D, G>(blk, sm, bv, t0, w, lane);
  }
  asm volatile("" ::: "memory");
}

// The walk itself.  K and V of the unit after the current one are requested
// while the current one is being computed.  t/phys_u/sc hold the first unit
// (already requested by the caller), hb the header batch of walk units 0..63.
template <int D, int G, int BITS>
__device__ __forceinline__ void dense_units(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const DecodeParams& p, int b, int h, int split,
                            int units, int n_cold, int w, int lane, Tiles<D, BITS>& t, int phys_u, float2 sc, int hb) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  const CacheView& c = p.c;
  const int CU = p.units_per_split;
  const int stride = p.nsplit * CU;
  int run0 = split * CU;
  int run_end = min(units, run0 + CU);
  int u = run0 + w < units ? run0 + w : -1;
  // next unit of this wave after x (x is the most recent unit handed out)
  auto advance = [&](int x) -> int {
    int nx = x + kWaves;
    if (nx < run_end) return nx;
    run0 += stride;
    run_end = min(units, run0 + CU);
    nx = run0 + w;
    return nx < units ? nx : -1;
  };
  int kb = 0;  // walk index of lane 0 of the header batch
  auto phys_of = [&](int k) -> int {
    if (k - kb >= 64) {
      kb = k;
      hb = header_batch(c, b, kb, split, p.nsplit, CU, w, lane);
    }
    return __builtin_amdgcn_readlane(hb, k - kb);
  };
  const __amdgpu_buffer_rsrc_t rs = scales_rsrc(c);
  int k = 0;
  int un = u >= 0 ? advance(u) : -1;
  int phys_n = un >= 0 ? phys_of(k + 1) : -1;
  while (u >= 0) {
    const int nv = phys_u >= 0 ? min(S, n_cold - u * S) : 0;
    const __amdgpu_buffer_rsrc_t rn = tile_rsrc<D, BITS>(c, phys_n, h);  // empty when there is no next unit
    float4_t s[C::NQ];
    qk_codes_refill<D, G, BITS>(t.kr, sm, lane, s, rn);
    float alpha[C::NG], coef[C::NG];
    softmax_unit<D, G, false>(st, sm, s, lane < nv, sc.x * p.qscale, 1.f, sc.y, alpha, coef, w, lane);
    sc = load_scales(rs, phys_n, c.H, h);  // the scale pair is free once the softmax has used it
    BlockAcc<D, G> blk;
    pv_dense_refill<D, G, BITS>(blk, sm, t.vr, w, lane, rn);
    fold_block<D, G>(st, blk, alpha, coef);
    wave_lds_sync();  // this unit's weight reads are done before the next unit's writes
    u = un;
    phys_u = phys_n;
    ++k;
    if (u >= 0) {
      un = advance(u);
      phys_n = un >= 0 ? phys_of(k + 1) : -1;
    }
  }
}

// The walk with dynamic unit claims (long resident splits).  Splits that
// stream the same number of blocks were measured to finish up to 6x apart
// (memory bandwidth is not shared evenly between workgroups), so after its
// first unit (split * 4 + w, static: the first memory round needs no claim)
// each wave claims units from the (sequence, kv-head) counter: unit =
// base + claim (base = 4 x the splits of this (sequence, kv-head), past every
// static first unit), until a claim lands past the last unit.  Every unit is
// claimed exactly once and computed by the wave that claimed it.  Claims run
// two units ahead: while unit u is computed, the tiles of the next unit are
// requested (as in the static walk), and the claim for the unit after it is
// resolved and its header requested.
// t/phys_u/sc hold the first unit (requested by the caller), un/hn the next
// unit and its pending header load (un < 0: none), cl the pending claim for
// the unit after it (valid when un >= 0).
template <int D, int G, int BITS>
__device__ __forceinline__ void dense_units_claim(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const DecodeParams& p, int b, int h,
                                  int bh, int units, int base, int n_cold, int w, int lane, Tiles<D, BITS>& t, int u,
                                  int phys_u, float2 sc, int un, int hn, unsigned cl) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  const CacheView& c = p.c;
  unsigned* work = p.work + static_cast<size_t>(bh) * kClaimStride;
  const __amdgpu_buffer_rsrc_t rs = scales_rsrc(c);
  int phys_n = un >= 0 ? header_phys(c, hn) : -1;
  while (u >= 0) {
    const int nv = phys_u >= 0 ? min(S, n_cold - u * S) : 0;
    const __amdgpu_buffer_rsrc_t rn = tile_rsrc<D, BITS>(c, phys_n, h);  // empty when there is no next unit
    float4_t s[C::NQ];
    qk_codes_refill<D, G, BITS>(t.kr, sm, lane, s, rn);
    float alpha[C::NG], coef[C::NG];
    softmax_unit<D, G, false>(st, sm, s, lane < nv, sc.x * p.qscale, 1.f, sc.y, alpha, coef, w, lane);
    sc = load_scales(rs, phys_n, c.H, h);
    // the unit after next: resolve its claim, request its header
    int un2 = -1, hn2 = -1;
    if (un >= 0) {
      un2 = base + static_cast<int>(__builtin_amdgcn_readfirstlane(cl));
      if (un2 >= units) un2 = -1;
      else hn2 = header_load(c, b, un2);
    }
    BlockAcc<D, G> blk;
    pv_dense_refill<D, G, BITS>(blk, sm, t.vr, w, lane, rn);
    fold_block<D, G>(st, blk, alpha, coef);
    wave_lds_sync();
    u = un;
    phys_u = phys_n;
    un = un2;
    if (un >= 0) {
      phys_n = header_phys(c, hn2);
      cl = claim_issue(work, lane);
    } else {
      phys_n = -1;
    }
  }
}

// ---------------------------------------------------------------- sparse units
// Up to kSparseUnit selected cold tokens, one per lane (lanes past the unit are
// masked).  Once the tokens' physical blocks are known, all of the unit's
// memory traffic is issued in one round: the K rows and block scales (lane =
// token) and, for PV, the value codes of every token at the lane's channels
// (lane c: channels c and 64 + c), read through a per-token buffer descriptor
// that is empty for a masked token.  Each token has its own block scales: the
// logit scale is per lane, and the value weight is taken relative to the
// largest V scale of the unit (vcoef).
// The lane's selection entry of a sparse unit (-1 past the unit or the list).
__device__ __forceinline__ int sel_entry(const int32_t* sel_bh, int k_sel, int unit, int lane) {
  const int e = unit * kSparseUnit + lane;
  return (lane < kSparseUnit && e < k_sel) ? sel_bh[e] : -1;
}

// Value element of token tt (row of a V tile) at channel c, as the bits of the tile format: an
// 8-bit code byte, a 4-bit offset-binary nibble or an fp16 value (b8/b16 buffer loads; an empty
// descriptor reads 0).
template <int D, int BITS>
__device__ __forceinline__ uint32_t v_element(__amdgpu_buffer_rsrc_t r, int tt, int c) {
  using F = Fmt<BITS>;
  constexpr int TB = F::template tile_bytes<D>();
  constexpr int E = F::kElems;
  const int chunk = TB + ((tt / E) * D + c) * 16;
  if constexpr (BITS == 8) return __builtin_amdgcn_raw_buffer_load_b8(r, chunk + tt % E, 0, 0);
  else if constexpr (BITS == 4) return __builtin_amdgcn_raw_buffer_load_b8(r, chunk + nib_byte(tt % E), 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b16(r, chunk + (tt % E) * 2, 0, 0);
}

// Exact PV operand of four gathered tokens from their value elements (v_element of each, and for
// 4-bit tiles the token index, which names the nibble of the loaded byte).
template <int BITS>
__device__ __forceinline__ half4_t gathered_operand(const uint32_t (&e)[4], const int (&tt)[4]) {
  if constexpr (BITS == 8) {
    return codes_to_half4(e[0] | (e[1] << 8) | (e[2] << 16) | (e[3] << 24));
  } else if constexpr (BITS == 4) {
    uint32_t n[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) n[i] = (e[i] >> nib_shift(tt[i] % Fmt<4>::kElems)) & 0xFu;
    const half2_t off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    const half2_t a = __builtin_bit_cast(half2_t, 0x64006400u | n[0] | (n[1] << 16)) - off;
    const half2_t b = __builtin_bit_cast(half2_t, 0x64006400u | n[2] | (n[3] << 16)) - off;
    return half4_t{a.x, a.y, b.x, b.y};
  } else {
    const half2_t a = __builtin_bit_cast(half2_t, e[0] | (e[1] << 16));
    const half2_t b = __builtin_bit_cast(half2_t, e[2] | (e[3] << 16));
    return half4_t{a.x, a.y, b.x, b.y};
  }
}

// idx: the lane's selection entry (sel_entry of this unit).
template <int D, int G, int BITS>
__device__ __forceinline__ void gather_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, int idx, int b, int h,
                            int n_cold, float qscale, int w, int lane) {
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
  constexpr int S = kBlockSize;
  constexpr int TU = kSparseUnit;
  constexpr int TB = F::template tile_bytes<D>();
  static_assert(TU % 4 == 0 && TU <= 64, "whole PV steps of 4 tokens, one token per lane");
  int phys = -1;
  if (idx >= 0 && idx < n_cold) {
    const int j = idx / S;
    if (j < c.max_blocks) phys = c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
  }
  const bool valid = phys >= 0 && phys < c.num_phys;
  if (__ballot(valid) == 0) return;  // no token: the state is unchanged (also: num_phys may be 0)
  const int t = valid ? idx % S : 0;
  // K row and scales of the lane's token; a masked lane reads block 0 (present: some token is
  // valid) and its values are discarded
  const int pl = valid ? phys : 0;
  const uint4* tk = reinterpret_cast<const uint4*>(c.cold + tile_offset(pl, h, 0, c.H, TB));
  uint4 kr[D / F::kElems];
#pragma unroll
  for (int ch = 0; ch < D / F::kElems; ++ch) kr[ch] = tk[ch * S + t];
  const float2 scl = *reinterpret_cast<const float2*>(c.scales + (static_cast<size_t>(pl) * c.H + h) * 2);
  // value elements: token k of the unit at channel 64 ps + lane
  const int pm = valid ? phys : -1;
  uint32_t vb[TU][C::NDL];
  int tts[TU];
#pragma unroll
  for (int k = 0; k < TU; ++k) {
    const int pk = __builtin_amdgcn_readlane(pm, k);
    const int tt = __builtin_amdgcn_readlane(t, k);
    tts[k] = tt;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<D, BITS>(c, pk, h);  // empty for a masked token: reads 0
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) vb[k][ps] = v_element<D, BITS>(r, tt, 64 * ps + lane);
  }
  const float2 sc = valid ? scl : make_float2(0.f, 0.f);
  float4_t s[C::NQ];
  qk_codes<D, G, BITS>(kr, sm, lane, s);
  const float vmax = wave_max_dpp(sc.y);
  const float vw = vmax > 0.f ? sc.y * __builtin_amdgcn_rcpf(vmax) : 0.f;
  float alpha[C::NG], coef[C::NG];
  softmax_unit<D, G, true>(st, sm, s, valid, sc.x * qscale, vw, vmax, alpha, coef, w, lane);
  BlockAcc<D, G> blk;
  zero_blk<D, G>(blk);
#pragma unroll
  for (int t0 = 0; t0 < TU; t0 += 4) {
    half4_t bv[C::NDL];
    const int tq[4] = {tts[t0], tts[t0 + 1], tts[t0 + 2], tts[t0 + 3]};
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) {
      const uint32_t e[4] = {vb[t0][ps], vb[t0 + 1][ps], vb[t0 + 2][ps], vb[t0 + 3][ps]};
      bv[ps] = gathered_operand<BITS>(e, tq);
    }
    pv_step<D, G>(blk, sm, bv, t0, w, lane);
  }
  fold_block<D, G>(st, blk, alpha, coef);
  wave_lds_sync();
}

// ---------------------------------------------------------------- compacted store units
// Unit u (64 stored tokens) of a (sequence, kv-head) of a compacted sparse store: a K tile and a V
// tile in the cold-block chunk layouts, read like a dense block, and each token's own (K, V) scales
// (lane = token).  The logit scale is per lane and the value weight is taken relative to the unit's
// largest V scale, as for gathered tokens.  count: the stored tokens of the (sequence, kv-head).
// Request unit u's tiles (an empty descriptor past the store's units: the loads return 0) and the
// lane's token scales.
template <int D, int BITS>
__device__ __forceinline__ void store_issue(const DecodeParams& p, int bh, int u, int lane, Tiles<D, BITS>& t,
                                            float2& sc) {
  constexpr int S = kBlockSize;
  constexpr int E = Fmt<BITS>::kElems;
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  const bool ok = u < p.store_units;
  const size_t unit = static_cast<size_t>(bh) * p.store_units + (ok ? u : 0);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(p.store_units_base + unit * 2 * TB, ok ? 2u * TB : 0u);
  issue_k<D, BITS>(t, r, lane);
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
#pragma unroll
  for (int ps = 0; ps < D / 64; ++ps)
#pragma unroll
    for (int vc = 0; vc < S / E; ++vc) t.vr[ps][vc] = load_stream_buf(r, lo + TB + (vc * D + 64 * ps) * 16);
  const float2 v = p.store_scales[unit * S + opaque_index(lane)];  // (unit 0 of the pair when !ok: in bounds)
  sc = make_float2(ok ? v.x : 0.f, ok ? v.y : 0.f);
}

// Attend unit u from its requested tiles and the lane's token scales; count: the stored tokens of the
// (sequence, kv-head).
template <int D, int G, int BITS>
__device__ __forceinline__ void store_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const DecodeParams& p, int u, int count,
                           const Tiles<D, BITS>& t, float2 sc, int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  const bool valid = lane < count - u * S;
  float4_t s[C::NQ];
  qk_codes<D, G, BITS>(t.kr, sm, lane, s);
  const float sv = valid ? sc.y : 0.f;
  const float vmax = wave_max_dpp(sv);
  const float vw = vmax > 0.f ? sv * __builtin_amdgcn_rcpf(vmax) : 0.f;
  float alpha[C::NG], coef[C::NG];
  softmax_unit<D, G, true>(st, sm, s, valid, sc.x * p.qscale, vw, vmax, alpha, coef, w, lane);
  BlockAcc<D, G> blk;
  pv_dense<D, G, BITS>(blk, sm, t.vr, w, lane);
  fold_block<D, G>(st, blk, alpha, coef);
  wave_lds_sync();
}

// Partials are exchanged between workgroups that may sit on different XCDs
// (each with its own L2).  They are written and read with agent-scope relaxed
// atomic accesses (device-coherent sc1 loads/stores, 8 bytes each), so
// publishing them needs only a wait for the stores to complete, not an
// L2-wide writeback.
__device__ __forceinline__ void store_coherent2(float* p, float a, float b) {
  const uint64_t v = static_cast<uint64_t>(__builtin_bit_cast(uint32_t, a)) |
                     (static_cast<uint64_t>(__builtin_bit_cast(uint32_t, b)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_coherent2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__builtin_bit_cast(float, static_cast<uint32_t>(v)),
                     __builtin_bit_cast(float, static_cast<uint32_t>(v >> 32)));
}

// Partial record of one split: m (base-2 log units), l, z (sum of weight * base-2 logit), 0 and
// acc[D] for each of the G query heads; records are 16-byte aligned (D + 4 is a multiple of 4).
template <int D>
__device__ __forceinline__ float* partial_ptr(const DecodeParams& p, int bh, int split, int g) {
  return p.partials + ((static_cast<size_t>(bh) * p.nparts + split) * p.G + g) * (D + kRecHead);
}

// Query rows of one kv-head's group into LDS as fp16 (exact), 16 bytes per
// thread in one round; rows past G are zero.
template <int D, int G>
__device__ __forceinline__ void copy_query(const _Float16* qg, _Float16 (*qh)[4][Cfg<D, G>::QROW], int tid) {
  using C = Cfg<D, G>;
  constexpr int VPR = D / 8;
  for (int i = tid; i < 4 * C::NQ * VPR; i += kThreads) {
    const int g = i / VPR, v = i % VPR;
    const uint4 val = g < G ? reinterpret_cast<const uint4*>(qg + static_cast<size_t>(g) * D)[v] : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&qh[g / 4][g % 4][v * 8]) = val;
  }
}

// Units one (sequence, kv-head) attends in its cold splits: stored units (compacted store), sparse
// units of the selection, or cold blocks (the fused step: the full blocks before the tail block).
template <int MODE, bool FUSED>
__device__ __forceinline__ int pair_units(const DecodeParams& p, int n_seq, int store_count) {
  const SeqGeom sg = seq_geom(n_seq, p.c.T, kBlockSize);
  // (a store holds at most store_units units per (sequence, kv-head): a count from a store built for
  // another width never walks past it)
  if (MODE == kModeStore) return min(cdiv(max(store_count, 0), kBlockSize), p.store_units);
  if (sg.n_cold <= 0) return 0;
  return MODE == kModeGather ? cdiv(p.k_sel, kSparseUnit) : (FUSED ? sg.n_cold / kBlockSize : sg.n_blk);
}

// Cold splits taking part for a (sequence, kv-head) of `units` units (see table_splits).
__device__ __forceinline__ int splits_of_pair(const DecodeParams& p, int units) {
  return p.wg_order == kOrderTable ? table_splits(p.nsplit, p.units_per_split, units) : p.nsplit;
}

// ---- cold split: stream its units, merge the 4 waves, write the partial
template <int D, int G, int BITS, int MODE, bool FUSED, bool CLAIM, bool STATS>
__device__ __forceinline__ void cold_split(const DecodeParams& p, DecodeSmem<D, G>& sm, int b, int h, int bh, int split,
                                           int n_host) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  constexpr int NG = C::NG;
  const CacheView& c = p.c;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the length, this wave's first header and (dense) its first tiles are requested together
  // with the query copy; the tiles are used only if the unit exists
  // first memory round: the query rows, the length and this wave's header batch; the first
  // unit's tiles follow as soon as its physical block id is known
  constexpr int QITEMS = 4 * C::NQ * (D / 8);  // 16-byte query vectors (rows past G are zero)
  constexpr int QPT = (QITEMS + kThreads - 1) / kThreads;
  const _Float16* qg = p.q + (static_cast<size_t>(b) * c.H * G + static_cast<size_t>(h) * G) * D;
  u32x4_t qv[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {  // unconditional loads (clamped item), zero outside the rows
    const int i = tid + k * kThreads;
    const int g = i / (D / 8);
    const bool ok = i < QITEMS && g < G;
    const u32x4_t v = reinterpret_cast<const u32x4_t*>(qg)[ok ? i : 0];
    qv[k] = ok ? v : u32x4_t{0u, 0u, 0u, 0u};
  }
  // needed only after the barrier: kept in a vector register, waited for there (issued before the
  // tiles, so that wait does not include them); a fused step's length from the launch arguments
  const int n_seq_lane = n_host >= 0 ? n_host : c.seq_len[opaque_index(b)];
  Tiles<D, BITS> t0;
  float2 sc0 = make_float2(0.f, 0.f);
  int phys0 = -1, hb = -1;
  constexpr bool SPARSE = MODE == kModeGather;
  const int32_t* sel_bh = SPARSE ? p.sel + static_cast<size_t>(bh) * p.k_sel : nullptr;
  // store mode: the (sequence, kv-head)'s stored token count, with the first round
  const int count_lane = MODE == kModeStore ? p.store_counts[opaque_index(bh)] : 0;
  int sel0 = -1;  // sparse: this wave's first unit's selection entry, requested with the query
  unsigned cl0 = 0;  // claim walk: the first claim
  if (SPARSE) {
    sel0 = sel_entry(sel_bh, p.k_sel, split * p.units_per_split + w, lane);
  } else if constexpr (MODE == kModeStore) {
    // the first unit's tiles and scales travel with the first round (their addresses do not
    // depend on the stored count)
    store_issue<D, BITS>(p, bh, split * p.units_per_split + w, lane, t0, sc0);
  } else if constexpr (CLAIM) {
    // claim walk: the first unit is split * 4 + w; the first claim travels with the first round
    hb = header_load(c, b, split * kWaves + w);
    cl0 = claim_issue(p.work + static_cast<size_t>(bh) * kClaimStride, lane);
    phys0 = header_phys(c, hb);
    const __amdgpu_buffer_rsrc_t r0 = tile_rsrc<D, BITS>(c, phys0, h);
    issue_k<D, BITS>(t0, r0, lane);
    issue_v<D, BITS>(t0, sc0, r0, scales_rsrc(c), phys0, c.H, h, lane);
  } else {
    hb = header_batch(c, b, 0, split, p.nsplit, p.units_per_split, w, lane);
    phys0 = __builtin_amdgcn_readlane(hb, 0);
    const __amdgpu_buffer_rsrc_t r0 = tile_rsrc<D, BITS>(c, phys0, h);
    issue_k<D, BITS>(t0, r0, lane);
    issue_v<D, BITS>(t0, sc0, r0, scales_rsrc(c), phys0, c.H, h, lane);
  }
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * kThreads;
    if (i < QITEMS) *reinterpret_cast<u32x4_t*>(&sm.qh[i / (D / 8) / 4][i / (D / 8) % 4][(i % (D / 8)) * 8]) = qv[k];
  }
  __syncthreads();

  const SeqGeom sg = seq_geom(__builtin_amdgcn_readfirstlane(n_seq_lane), c.T, S);
  // fused append: only the full blocks before the one the appended token spills into (n_cold is
  // the count before the append, so the block holding cold token n_cold is excluded)
  const int store_count = MODE == kModeStore ? __builtin_amdgcn_readfirstlane(count_lane) : 0;
  const int units = pair_units<MODE, FUSED>(p, sg.n, store_count);

  WaveState<D, G> st;
  st.stats = STATS;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    st.m[g] = kNegInf;
    st.l[g] = 0.f;
    if (st.stats) z_lane(sm, w, g, lane) = 0.f;
    float qs = 0.f;
#pragma unroll
    for (int k = lane; k < D; k += 64) qs += static_cast<float>(sm.qh[g / 4][g % 4][k]);
    st.qb[g] = Fmt<BITS>::kBias * wave_sum_dpp(qs);
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) st.acc[quad][ps] = float4_t{0.f, 0.f, 0.f, 0.f};

  if (SPARSE) {
    const int CU = p.units_per_split;
    for (int run = split; run * CU < units; run += p.nsplit) {
      const int u_end = min(units, (run + 1) * CU);
      for (int u = run * CU + w; u < u_end; u += kWaves) {
        const int idx = (run == split && u == run * CU + w) ? sel0 : sel_entry(sel_bh, p.k_sel, u, lane);
        gather_unit<D, G, BITS>(st, sm, c, idx, b, h, sg.n_cold, p.qscale, w, lane);
      }
    }
  } else if constexpr (MODE == kModeStore) {
    const int CU = p.units_per_split;
    for (int run = split; run * CU < units; run += p.nsplit) {
      const int u_end = min(units, (run + 1) * CU);
      for (int u = run * CU + w; u < u_end; u += kWaves) {
        if (run != split || u != run * CU + w) store_issue<D, BITS>(p, bh, u, lane, t0, sc0);
        store_unit<D, G, BITS>(st, sm, p, u, store_count, t0, sc0, w, lane);
      }
    }
  } else if constexpr (CLAIM) {
    const int u0 = split * kWaves + w;
    int un = -1, hn = -1;
    unsigned cl = 0;
    // claims start past the static first units of this (sequence, kv-head)'s splits
    const int base = splits_of_pair(p, units) * kWaves;
    if (u0 < units) {  // else units <= base: every claim lands past the last unit
      un = base + static_cast<int>(__builtin_amdgcn_readfirstlane(cl0));
      if (un >= units) {
        un = -1;
      } else {
        hn = header_load(c, b, un);
        cl = claim_issue(p.work + static_cast<size_t>(bh) * kClaimStride, lane);
      }
    }
    dense_units_claim<D, G, BITS>(st, sm, p, b, h, bh, units, base, sg.n_cold, w, lane, t0, u0 < units ? u0 : -1, phys0,
                                  sc0, un, hn, cl);
  } else {
    dense_units<D, G, BITS>(st, sm, p, b, h, split, units, sg.n_cold, w, lane, t0, phys0, sc0, hb);
  }
  // merge the 4 waves: lane holds out[4quad + r][64 pass + lane]
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float lsum = wave_sum_dpp(st.l[g]);
    const float zsum = st.stats ? wave_sum_dpp(z_lane(sm, w, g, lane)) : 0.f;
    if (lane == 0) {
      sm.wm[w][g] = st.m[g];
      sm.wl[w][g] = lsum;
      sm.wz[w][g] = zsum;
    }
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.wacc[w][4 * quad + r][64 * ps + lane] = st.acc[quad][ps][r];
  __syncthreads();
  for (int idx = tid; idx < G * (D / 2); idx += kThreads) {
    const int g = idx / (D / 2), d = 2 * (idx % (D / 2));
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.wm[ww][g]);
    float L = 0.f, Z = 0.f, A0 = 0.f, A1 = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if (sm.wm[ww][g] == kNegInf) continue;
        const float f = exp2_approx(sm.wm[ww][g] - M);
        const float2 a = *reinterpret_cast<const float2*>(&sm.wacc[ww][g][d]);
        L = fmaf(f, sm.wl[ww][g], L);
        Z = fmaf(f, sm.wz[ww][g], Z);
        A0 = fmaf(f, a.x, A0);
        A1 = fmaf(f, a.y, A1);
      }
    }
    float* pg = partial_ptr<D>(p, bh, split, g);
    store_coherent2(pg + kRecHead + d, A0, A1);
    if (d == 0) {
      store_coherent2(pg, M, L);
      store_coherent2(pg + 2, Z, 0.f);
    }
  }
}

// ---- hot zone: the FP16 ring (Hybrid KV Cache page 2.1: the most recent
// tokens in full precision).  Chunks of kHotChunk slots are staged through LDS
// with coalesced loads; wave 0 computes the logits with the same MFMA as the
// cold blocks (lane = slot, fp16 K rows are already MFMA operands) and the
// softmax weights; all four waves then accumulate thread (g, d) = sum_t p v.
// Attends ring slots [0, n_hot); slot sub_slot (if >= 0) is read from the
// rows sub_k / sub_v instead of the ring (the token a fused append is putting
// there).  The first chunk's loads are issued ahead of the query's, so both
// take one memory round trip.  Leaves m, l (base-2 units) and acc in hm.
template <int D, int G>
__device__ void hot_attend(const DecodeParams& p, HotSmem<D, G>& hm, _Float16 (*qh)[4][Cfg<D, G>::QROW], int b, int h,
                           int bh, int n_hot, int sub_slot, const _Float16* sub_k, const _Float16* sub_v) {
  using C = Cfg<D, G>;
  constexpr int NG = 4 * C::NQ;
  constexpr int ROW = 2 * D + 8;          // padded fp16 [K|V] row
  constexpr int VPR = 2 * D / 8;          // 16-byte vectors per row
  constexpr int NV = (kHotChunk * VPR + kThreads - 1) / kThreads;
  const CacheView& c = p.c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const _Float16* hot_bh = c.hot + static_cast<size_t>(bh) * c.T * 2 * D;
  static_assert(kHotChunk * VPR % kThreads == 0, "a chunk is a whole number of vectors per thread");
  // this thread's vectors of the chunk at `base`, loaded without branches (a branch would merge the
  // loaded value at its join and wait there): rows past the window read the chunk's row 0, which the
  // ring always holds, and are zeroed when staged
  auto load_chunk = [&](int base, uint4 (&buf)[NV]) {
    const uint4* src = reinterpret_cast<const uint4*>(hot_bh + static_cast<size_t>(base) * 2 * D);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = tid + k * kThreads;
      const int r = i / VPR, v = i % VPR;  // row, and vector of its K row then V row
      const uint4* ptr = base + r == sub_slot ? reinterpret_cast<const uint4*>(v < D / 8 ? sub_k : sub_v) + v % (D / 8)
                                              : src + (base + r < n_hot ? i : v);
      buf[k] = *ptr;
    }
  };
  float m[NG], l[NG];  // wave 0's running softmax state (wave-uniform)
  const bool stats = p.c.entropy != nullptr;  // entropy statistic asked for: its sum runs in hm.zs
  // one chunk: stage it (with the query on the first), logits and weights by wave 0, then every
  // thread's share of acc
  auto attend_chunk = [&](int base, const uint4 (&buf)[NV]) {
    const int cnt = min(kHotChunk, n_hot - base);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = tid + k * kThreads;
      *reinterpret_cast<uint4*>(&hm.kv[(i / VPR) * ROW + (i % VPR) * 8]) = i / VPR < cnt ? buf[k] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    if (w == 0) {
      const bool valid = lane < cnt;
      const _Float16* kr = &hm.kv[(valid ? lane : 0) * ROW];
      float4_t s[C::NQ];
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) s[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int k0 = 0; k0 < D; k0 += 4) {
        const half4_t bk = *reinterpret_cast<const half4_t*>(kr + k0);
#pragma unroll
        for (int quad = 0; quad < C::NQ; ++quad)
          s[quad] = mfma_qk(*reinterpret_cast<const half4_t*>(&qh[quad][lane & 3][k0]), bk, s[quad]);
      }
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int g = 4 * quad + r;
          const float z = valid ? s[quad][r] * p.qscale : kNegInf;
          const float mn = fmaxf(m[g], wave_max_dpp(z));
          const float alpha = exp2_approx(m[g] - mn);
          const float pt = valid ? exp2_approx(z - mn) : 0.f;
          l[g] = l[g] * alpha + wave_sum_dpp(pt);
          if (stats) {
            const float zsum = wave_sum_dpp(valid ? pt * z : 0.f);
            if (lane == 0) hm.zs[g] = fmaf(hm.zs[g], alpha, zsum);
          }
          m[g] = mn;
          if (lane < kHotChunk) hm.z[g][lane] = pt;
          if (lane == 0) hm.alpha[g] = alpha;
        }
      }
    }
    __syncthreads();
    // thread (g, d): channels d, d + 1 of query head g over every staged row, a fixed count so that
    // the LDS reads are issued together (rows past cnt are zero with weight 0: fma(0, 0, a) = a)
    for (int i = tid; i < G * (D / 2); i += kThreads) {
      const int g = i / (D / 2), d = 2 * (i % (D / 2));
      float a0 = hm.acc[g][d] * hm.alpha[g], a1 = hm.acc[g][d + 1] * hm.alpha[g];
#pragma unroll
      for (int t = 0; t < kHotChunk; ++t) {
        const float z = hm.z[g][t];
        const uint32_t v2 = *reinterpret_cast<const uint32_t*>(&hm.kv[t * ROW + D + d]);
        a0 = fmaf(z, half_lo(v2), a0);
        a1 = fmaf(z, half_hi(v2), a1);
      }
      hm.acc[g][d] = a0;
      hm.acc[g][d + 1] = a1;
    }
    __syncthreads();
  };
  // the first chunk's loads and the query's go out together (straight-line code: one round trip)
  uint4 buf[NV];  // all of a chunk's loads in flight together
  load_chunk(0, buf);
  copy_query<D, G>(p.q + (static_cast<size_t>(b) * c.H * G + static_cast<size_t>(h) * G) * D, qh, tid);
  for (int i = tid; i < G * D; i += kThreads) hm.acc[i / D][i % D] = 0.f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
  }
  if (tid < NG) hm.zs[tid] = 0.f;  // (wave 0, the only wave that updates it)
  if (n_hot > 0) attend_chunk(0, buf);
  for (int base = kHotChunk; base < n_hot; base += kHotChunk) {
    load_chunk(base, buf);
    attend_chunk(base, buf);
  }
  if (w == 0 && lane == 0) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      hm.m[g] = m[g];
      hm.l[g] = l[g];
    }
  }
  __syncthreads();
}

// The hot zone's partial record (split index nsplit).
template <int D, int G>
__device__ __forceinline__ void store_hot_partial(const DecodeParams& p, const HotSmem<D, G>& hm, int bh) {
  for (int i = threadIdx.x; i < G * (D / 2); i += kThreads) {
    const int g = i / (D / 2), d = 2 * (i % (D / 2));
    float* pg = partial_ptr<D>(p, bh, p.nsplit, g);
    store_coherent2(pg + kRecHead + d, hm.acc[g][d], hm.acc[g][d + 1]);
    if (d == 0) {
      store_coherent2(pg, hm.m[g], hm.l[g]);
      store_coherent2(pg + 2, hm.zs[g], 0.f);
    }
  }
}

// ---- hot split of a plain decode: the whole ring, partial at split index nsplit
template <int D, int G>
__device__ void hot_split(const DecodeParams& p, HotSmem<D, G>& hm, int b, int h, int bh) {
  const SeqGeom sg = seq_geom(p.c.seq_len[b], p.c.T, kBlockSize);
  hot_attend<D, G>(p, hm, hm.qh, b, h, bh, sg.n_hot, -1, nullptr, nullptr);
  store_hot_partial<D, G>(p, hm, bh);
}

// ---- fused one-token append (hkv_append_decode): one more workgroup per
// (sequence, kv-head) next to the cold splits, with two partial records.
//   The new hot window (split index nsplit): ring slots [0, min(n0 + 1, T))
//     with the new token's slot read from k_new / v_new (it never reads that
//     slot from the ring, which the append overwrites).
//   The append itself (split index nsplit + 1; Hybrid KV Cache page 2.1 /
//     4.2: the token leaving the hot zone joins the cold zone, quantised with
//     its block's scale) and the attention over that tail block jt.  The
//     spilled token becomes row ts of block jt, re-coded exactly as the
//     standalone append codes it (only the new row while the block maximum is
//     unchanged, else the whole block from its FP16 tail-shadow rows); the
//     tail shadow, the header and the ring slot are written.  The block's tile
//     registers for the attention come from this workgroup's own codes in LDS
//     (every row is coded there; with an unchanged maximum they equal the
//     stored codes), so nothing waits for the code stores.  The cold splits
//     cover only the full blocks before jt.
// The hot window goes first, in the LDS the block's codes take afterwards; its loads are issued
// behind the append's first round, so the two share one memory round trip.

template <int D, int G, int BITS>
struct AppendSmem {
  static constexpr int EB = BITS == 0 ? 2 : 1;       // stage bytes per element: one code, or one fp16 value
  static constexpr int KROW = D * EB + 16;           // K stage row: one token's channels (padded)
  static constexpr int VROW = kBlockSize * EB + 16;  // V stage row: one channel's tokens (padded)
  struct Stage {
    alignas(16) int8_t k[kBlockSize * KROW];         // the block's K codes / values, [token][channel]
    alignas(16) int8_t v[D * VROW];                  // its V codes / values, [channel][token]
  };
  DecodeSmem<D, G> unit;                             // tail block jt, attended by wave 0
  union {
    Stage stage;                                     // from the coding on
    HotSmem<D, G> hot;                               // the hot window, attended before the coding
  };
  float red[4][kWaves];
  float rerr[2][kWaves];                             // debug statistic: per-wave largest |x - code * scale|
};

template <int D, int G, int BITS, bool STATS>
__device__ void append_unit_split(const DecodeParams& p, AppendSmem<D, G, BITS>& am, int b, int h, int bh, int n_host) {
  __builtin_amdgcn_s_setprio(3);  // the append's coding and its block's attention sit on the step's critical path
  using C = Cfg<D, G>;
  using F = Fmt<BITS>;
  using AS = AppendSmem<D, G, BITS>;
  constexpr int S = kBlockSize;
  constexpr int TPT = kThreads / S;     // threads per token row
  constexpr int CPT = D / TPT;          // channels per thread
  constexpr int NV = CPT / 8;           // 16-byte vectors per thread and row
  constexpr int KROW = AS::KROW;
  constexpr int VROW = AS::VROW;
  constexpr int EB = AS::EB;
  constexpr int E = F::kElems;
  constexpr int TB = F::template tile_bytes<D>();
  constexpr int VR = D / 8;             // 16-byte vectors per fp16 row
  constexpr int NG = C::NG;
  const CacheView& c = p.c;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = c.T, H = c.H;
  const int t = tid / TPT, part = tid % TPT;
  const size_t bhs = static_cast<size_t>(bh);
  // length before the append: from the launch arguments, else from seq_len
  const int n0 = n_host >= 0 ? n_host : __builtin_amdgcn_readfirstlane(c.seq_len[b]);
  const bool spill = n0 >= T;
  const int ps = n0 - T;                   // the spilled token's position
  const int jt = spill ? ps / S : 0;
  const int ts = spill ? ps % S : 0;       // its row in block jt; rows below are already coded
  const int slot = n0 % T;                 // ring slot of the spilled token and of the new one
  const _Float16* knew = p.k_new + bhs * D;
  const _Float16* vnew = p.v_new + bhs * D;

  // ---- first round of loads: the spilled row, the block's old rows (tail shadow), its header and
  // the new token (the hot window's loads and the query's follow without a wait in between)
  // row t of block jt: an old row (t < ts, from the tail shadow), the spilled row (t == ts, from its
  // ring slot) or nothing; one slice per thread
  u32x4_t x[2][NV];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const u32x4_t* src = t < ts ? reinterpret_cast<const u32x4_t*>(c.tail + ((bhs * 2 + kv) * S + t) * D + part * CPT)
                                : reinterpret_cast<const u32x4_t*>(c.hot + ((bhs * T + slot) * 2 + kv) * D + part * CPT);
#pragma unroll
    for (int v = 0; v < NV; ++v) x[kv][v] = (spill && t <= ts) ? src[v] : u32x4_t{0u, 0u, 0u, 0u};
  }
  const int it = min(tid, 2 * VR - 1);  // new token: K row then V row, one vector per thread
  const u32x4_t nr = reinterpret_cast<const u32x4_t*>(it < VR ? knew : vnew)[it % VR];
  // the block's header: loaded now (from a clamped entry when the table has one) and resolved after
  // the hot window, so that waiting for it does not hold back the hot window's loads
  int ph_lane = -1;
  if (c.max_blocks > 0)
    ph_lane = c.headers[static_cast<size_t>(b) * c.max_blocks + min(jt, c.max_blocks - 1)].phys_block;
  // ---- the new hot window (partial nsplit), in the LDS the codes take next; it also puts the query
  // rows where the block attention reads them
  hot_attend<D, G>(p, am.hot, am.unit.qh, b, h, bh, min(n0 + 1, T), slot, knew, vnew);
  store_hot_partial<D, G>(p, am.hot, bh);
  const int ph = __builtin_amdgcn_readfirstlane(ph_lane);
  const int phys = spill && jt < c.max_blocks && ph >= 0 && ph < c.num_phys ? ph : -1;
  const bool stamp = p.stamps != nullptr;
  const unsigned long long t_hot = stamp ? __builtin_amdgcn_s_memrealtime() : 0ull;
  auto slice_max = [&](const u32x4_t (&x)[NV]) -> float { return slice_absmax<NV>(x); };
  const float m0 = slice_max(x[0]), m1 = slice_max(x[1]);
  float mx[4] = {t < ts ? m0 : 0.f, t < ts ? m1 : 0.f, t == ts ? m0 : 0.f, t == ts ? m1 : 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mx[i] = wave_max_dpp(mx[i]);
    if (lane == 0) am.red[i][w] = mx[i];
  }
  __syncthreads();  // also: the spilled slot has been read, it may be overwritten; the hot window's
                    // LDS has been read
  unsigned long long t_coded = 0ull;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = am.red[i][0];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) r = fmaxf(r, am.red[i][ww]);
    mx[i] = r;
  }

  // ---- codes of block jt (as the standalone append codes them).  Every row is coded into the
  // stage for the attention below: with an unchanged maximum the old rows' codes are the stored
  // ones (same FP16 values, same scale), and only row ts is written to memory; otherwise the
  // whole block is.  V codes are staged channel-major, as the tile stores them.  fp16 tiles stage
  // the values themselves (scale 1): the whole tile is written when the block opens (ts = 0),
  // afterwards only row ts.
  float scl[2] = {0.f, 0.f};  // the block's scales after the append
  bool whole[2] = {false, false};
  if (phys >= 0) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const float m_old = mx[kv], m_new = mx[2 + kv];
      if constexpr (BITS == 0) {
        whole[kv] = ts == 0;
        scl[kv] = 1.f;
        uint32_t* srow = reinterpret_cast<uint32_t*>(am.stage.k + t * KROW + part * CPT * 2);
        if (kv == 0) {
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) srow[4 * v + i] = x[0][v][i];
        } else {
#pragma unroll
          for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int cc = part * CPT + 8 * v + 2 * i;
              *reinterpret_cast<uint16_t*>(am.stage.v + cc * VROW + 2 * t) = static_cast<uint16_t>(x[1][v][i]);
              *reinterpret_cast<uint16_t*>(am.stage.v + (cc + 1) * VROW + 2 * t) = static_cast<uint16_t>(x[1][v][i] >> 16);
            }
        }
      } else {
        int8_t* tile = c.cold + tile_offset(phys, h, kv, H, TB);
        whole[kv] = !(ts > 0 && m_new <= m_old);
        const float sc = (whole[kv] ? fmaxf(m_old, m_new) : m_old) / static_cast<float>(F::kLimit);
        scl[kv] = sc;
        // branch-free: every value lies inside the scale's maximum, so the byte form needs no clamp
        const float rsc = quant_recip(sc);
        uint32_t qw[CPT / 4];
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i) {
          uint32_t cb[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = 4 * i + k;
            const uint32_t wd = x[kv][e / 8][(e % 8) / 2];
            cb[k] = code_bits(quant_quotient((e & 1) ? half_hi(wd) : half_lo(wd), sc, rsc));
          }
          qw[i] = pack_low_bytes(cb[0], cb[1], cb[2], cb[3]);
        }
        if (c.quant_err) {  // debug statistic: largest |x - code * scale| of the codes just made
          float err = 0.f;
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            const uint32_t wd = x[kv][e / 8][(e % 8) / 2];
            const float xv = (e & 1) ? half_hi(wd) : half_lo(wd);
            const float qv = static_cast<float>(static_cast<int8_t>(qw[e / 4] >> (8 * (e % 4))));
            err = fmaxf(err, __builtin_fabsf(fmaf(-qv, sc, xv)));
          }
          err = wave_max_dpp(err);
          if (lane == 0) am.rerr[kv][w] = err;
        }
        if (kv == 0) {
          uint32_t* srow = reinterpret_cast<uint32_t*>(am.stage.k + t * KROW + part * CPT);
#pragma unroll
          for (int i = 0; i < CPT / 4; ++i) srow[i] = qw[i];
        } else {
#pragma unroll
          for (int i = 0; i < CPT; ++i)
            am.stage.v[(part * CPT + i) * VROW + t] = static_cast<int8_t>(qw[i / 4] >> (8 * (i % 4)));
        }
        if (BITS == 8 && !whole[kv] && t == ts) {  // only row ts changes: write it in place
          if (kv == 0) {
#pragma unroll
            for (int ch = 0; ch < CPT / 16; ++ch)
              reinterpret_cast<uint4*>(tile)[((part * CPT) / 16 + ch) * S + t] =
                  make_uint4(qw[4 * ch] ^ kCodeOffsetWord, qw[4 * ch + 1] ^ kCodeOffsetWord,
                             qw[4 * ch + 2] ^ kCodeOffsetWord, qw[4 * ch + 3] ^ kCodeOffsetWord);
          } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i)
              tile[((t / 16) * D + part * CPT + i) * 16 + (t % 16)] =
                  static_cast<int8_t>((qw[i / 4] >> (8 * (i % 4))) ^ 0x80u);
          }
        }
      }
    }
    __syncthreads();  // stage complete
    if (stamp) t_coded = __builtin_amdgcn_s_memrealtime();
    if (tid < 2 && c.quant_err) {  // debug statistic: the block's largest |x - code * scale| (0 for fp16)
      float e = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) e = fmaxf(e, BITS == 0 ? 0.f : am.rerr[tid][ww]);
      c.quant_err[(static_cast<size_t>(phys) * H + h) * 2 + tid] = e;
    }
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      int8_t* tile = c.cold + tile_offset(phys, h, kv, H, TB);
      if (!whole[kv]) {
        if constexpr (BITS != 8) {
          // only row ts changes: its K chunks, and per channel the V bytes that hold it (4-bit: the
          // byte it shares with row ts + 4 or ts - 4 of its chunk word, rewritten from the stage)
          if (kv == 0) {
            if (tid < D / E)
              reinterpret_cast<uint4*>(tile)[tid * S + ts] = chunk_from_stage<BITS>(am.stage.k + ts * KROW + tid * E * EB);
          } else if (tid < D) {
            const int8_t* col = am.stage.v + tid * VROW;
            int8_t* chunk = tile + ((ts / E) * D + tid) * 16;
            if constexpr (BITS == 4) {
              const int r = ts % E;
              const int lo = ts - r + (r >> 3) * 8 + (r & 3);  // the byte's low-nibble row; its high one is lo + 4
              chunk[nib_byte(r)] = static_cast<int8_t>(((col[lo] & 0xF) ^ 8) | (((col[lo + 4] & 0xF) ^ 8) << 4));
            } else {
              *reinterpret_cast<uint16_t*>(chunk + (ts % E) * 2) = *reinterpret_cast<const uint16_t*>(col + 2 * ts);
            }
          }
        }
        continue;
      }
      constexpr int NVEC = TB / 16;
      for (int vi = tid; vi < NVEC; vi += kThreads) {
        uint4 out;
        if (kv == 0) {
          const int kc = vi / S, tt = vi % S;
          out = chunk_from_stage<BITS>(am.stage.k + tt * KROW + kc * E * EB);
        } else {
          const int vc = vi / D, cc = vi % D;
          out = chunk_from_stage<BITS>(am.stage.v + cc * VROW + vc * E * EB);
        }
        reinterpret_cast<uint4*>(tile)[vi] = out;
      }
      if (tid == 0) c.scales[(static_cast<size_t>(phys) * H + h) * 2 + kv] = scl[kv];
    }
    if (h == 0 && tid == 0) {
      hkv_block_header* hdr = c.headers + static_cast<size_t>(b) * c.max_blocks + jt;
      hdr->n_valid = ts + 1;
      hdr->logical_block = jt;
      hdr->flags = 0u;
    }
  }
  // FP16 shadow row of the still-partial block, and the new token into its ring slot
  if (spill && ts + 1 < S && t == ts) {
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(c.tail + ((bhs * 2 + kv) * S + t) * D + part * CPT);
#pragma unroll
      for (int v = 0; v < NV; ++v) dst[v] = x[kv][v];
    }
  }
  if (tid < 2 * VR)
    reinterpret_cast<u32x4_t*>(c.hot + ((bhs * T + slot) * 2 + tid / VR) * D)[tid % VR] = nr;

  const unsigned long long t_stored = stamp ? __builtin_amdgcn_s_memrealtime() : 0ull;
  // ---- tail block jt, rows [0, ts], by wave 0 with the cold-unit code
  if (w == 0) {
    float um[NG], ul[NG], uz[NG];
    float4_t uacc[C::NQ][C::NDL];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      um[g] = kNegInf;
      ul[g] = 0.f;
      uz[g] = 0.f;
    }
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
      for (int ps2 = 0; ps2 < C::NDL; ++ps2) uacc[quad][ps2] = float4_t{0.f, 0.f, 0.f, 0.f};
    if (phys >= 0) {
      // tile registers: K (lane = token) and V (lane = channel), from the stage
      Tiles<D, BITS> tl;
#pragma unroll
      for (int ch = 0; ch < D / E; ++ch) tl.kr[ch] = chunk_from_stage<BITS>(am.stage.k + lane * KROW + ch * E * EB);
#pragma unroll
      for (int ps2 = 0; ps2 < C::NDL; ++ps2)
#pragma unroll
        for (int vc = 0; vc < 64 / E; ++vc)
          tl.vr[ps2][vc] = chunk_from_stage<BITS>(am.stage.v + (64 * ps2 + lane) * VROW + vc * E * EB);
      WaveState<D, G> st;
      st.stats = STATS;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        st.m[g] = kNegInf;
        st.l[g] = 0.f;
        if (st.stats) z_lane(am.unit, 0, g, lane) = 0.f;
        float qs = 0.f;
#pragma unroll
        for (int k = lane; k < D; k += 64) qs += static_cast<float>(am.unit.qh[g / 4][g % 4][k]);
        st.qb[g] = F::kBias * wave_sum_dpp(qs);
      }
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
        for (int ps2 = 0; ps2 < C::NDL; ++ps2) st.acc[quad][ps2] = float4_t{0.f, 0.f, 0.f, 0.f};
      float4_t sq[C::NQ];
      qk_codes<D, G, BITS>(tl.kr, am.unit, lane, sq);
      float alpha[NG], coef[NG];
      softmax_unit<D, G, false>(st, am.unit, sq, lane <= ts, scl[0] * p.qscale, 1.f, scl[1], alpha, coef, 0, lane);
      BlockAcc<D, G> blk;
      pv_dense<D, G, BITS>(blk, am.unit, tl.vr, 0, lane);
      fold_block<D, G>(st, blk, alpha, coef);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        um[g] = st.m[g];
        ul[g] = wave_sum_dpp(st.l[g]);
        uz[g] = st.stats ? wave_sum_dpp(z_lane(am.unit, 0, g, lane)) : 0.f;
      }
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
        for (int ps2 = 0; ps2 < C::NDL; ++ps2) uacc[quad][ps2] = st.acc[quad][ps2];
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
      if (lane == 0) {
        am.unit.wm[0][g] = um[g];
        am.unit.wl[0][g] = ul[g];
        am.unit.wz[0][g] = uz[g];
      }
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
      for (int ps2 = 0; ps2 < C::NDL; ++ps2)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          am.unit.wacc[0][4 * quad + r][64 * ps2 + lane] = uacc[quad][ps2][r];
  }
  __syncthreads();
  if (stamp && tid == 0) {  // phase timestamps of this workgroup: hot window, codes, code stores, block attended
    const size_t wg = static_cast<size_t>(bh) * grid_parts(p) + p.nsplit;
    if (wg < static_cast<size_t>(p.stamp_wgs)) {
      unsigned long long* a = p.stamps + wg * 8;
      a[4] = t_hot;
      a[5] = t_coded;
      a[6] = t_stored;
      a[7] = __builtin_amdgcn_s_memrealtime();
    }
  }
  for (int i = tid; i < G * (D / 2); i += kThreads) {
    const int g = i / (D / 2), d = 2 * (i % (D / 2));
    float* pg = partial_ptr<D>(p, bh, p.nsplit + 1, g);
    store_coherent2(pg + kRecHead + d, am.unit.wacc[0][g][d], am.unit.wacc[0][g][d + 1]);
    if (d == 0) {
      store_coherent2(pg, am.unit.wm[0][g], am.unit.wl[0][g]);
      store_coherent2(pg + 2, am.unit.wz[0][g], 0.f);
    }
  }
}

// One launch per decode call: (nsplit + 1) x H x B workgroups; for each (sequence,
// kv-head) nsplit cold splits and one hot split (for a fused append, one workgroup with the hot
// window's and the tail block's records) write partial records, and the last of them to arrive
// merges all of them with the log-sum-exp rule (M = max m_s, L = sum e^(m_s - M) l_s,
// out = sum e^(m_s - M) acc_s / L) and writes the fp16 output.  Arrival is counted with a
// device-scope atomic in the workspace after the workgroup's record stores are complete; the
// merging workgroup resets it to zero.  The merge runs online over groups of kMergeChunk partials
// whose loads are all in flight together; thread i owns two adjacent output columns of one query
// head.
template <int D, int G, int BITS, int MODE, bool FUSED, bool CLAIM, bool STATS>
__device__ __forceinline__ void decode_body(const DecodeParams& p, const WgCoord wg, const int32_t* n0h = nullptr) {
  using AppendPart = typename std::conditional<FUSED, AppendSmem<D, G, BITS>, DecodeSmem<D, G>>::type;
  __shared__ union Smem {
    DecodeSmem<D, G> cold;
    HotSmem<D, G> hot;
    AppendPart app;
  } sm;
  __shared__ int s_last;
  const CacheView& c = p.c;
  const int split = wg.x;
  const int h = wg.y;
  const int b = wg.z;
  const int bh = b * c.H + h;
  const int tid = threadIdx.x;
  // a fused step's length before the append, from the launch arguments (-1: read seq_len)
  const int n_host = FUSED && n0h != nullptr ? n0h[b] : -1;
  // phase timestamps: this workgroup's 8 slots, when asked for and inside the buffer
  const size_t stamp_wg = static_cast<size_t>(bh) * grid_parts(p) + split;
  unsigned long long* const st = p.stamps && stamp_wg < static_cast<size_t>(p.stamp_wgs) ? p.stamps + stamp_wg * 8 : nullptr;
  const unsigned long long t_start = st ? __builtin_amdgcn_s_memrealtime() : 0ull;
  if (split < p.nsplit) {
    cold_split<D, G, BITS, MODE, FUSED, CLAIM, STATS>(p, sm.cold, b, h, bh, split, n_host);
  } else if constexpr (FUSED) {
    append_unit_split<D, G, BITS, STATS>(p, sm.app, b, h, bh, n_host);  // the hot window, then the append
  } else {
    hot_split<D, G>(p, sm.hot, b, h, bh);
  }
  // this (sequence, kv-head)'s unit count, for the number of its cold splits (loaded with the wait
  // for the partial stores)
  const int n_seq_lane = n_host >= 0 ? n_host : c.seq_len[opaque_index(b)];
  const int count_lane = MODE == kModeStore ? p.store_counts[opaque_index(bh)] : 0;
  // ---- arrival: wait until this workgroup's partial stores are complete, count, and let the
  // last workgroup merge
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t_done = st ? __builtin_amdgcn_s_memrealtime() : 0ull;
  __syncthreads();
  // partials of this (sequence, kv-head): its cold splits (records 0 .. ns_pair - 1), then the hot
  // zone's (and the tail block's) at nsplit (, nsplit + 1)
  const int ns_pair = splits_of_pair(p, pair_units<MODE, FUSED>(p, __builtin_amdgcn_readfirstlane(n_seq_lane),
                                                                 __builtin_amdgcn_readfirstlane(count_lane)));
  const int NS = ns_pair + (FUSED ? 2 : 1);
  const unsigned arrivals = FUSED && split >= p.nsplit ? 2u : 1u;  // the fused append's workgroup writes two
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&p.counters[bh], arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<unsigned>(NS) - arrivals;
  __syncthreads();
  if (st && tid == 0) {
    st[0] = t_start;
    st[1] = t_done;
    st[2] = __builtin_amdgcn_s_memrealtime();
    st[3] = 0ull;
  }
  if (!s_last) return;
  __builtin_amdgcn_s_setprio(3);  // the merge ends the (sequence, kv-head): ahead of streaming waves
  const int Hq = c.H * G;
  constexpr int REC = G * (D + kRecHead);  // floats per split record of one (sequence, kv-head)
  const float* base_bh = p.partials + static_cast<size_t>(bh) * p.nparts * REC;
  float* const entropy = c.entropy;
  for (int idx = tid; idx < G * (D / 2); idx += kThreads) {
    const int g = idx / (D / 2), d = 2 * (idx % (D / 2));
    const int off_ml = g * (D + kRecHead), off_a = off_ml + kRecHead + d;  // per lane; the split offset is uniform
    const bool want_z = entropy != nullptr && d == 0;  // the entropy statistic: the thread of column 0
    float M = kNegInf, L = 0.f, Z = 0.f, A0 = 0.f, A1 = 0.f;
    for (int s0 = 0; s0 < NS; s0 += kMergeChunk) {
      float2 ml[kMergeChunk], av[kMergeChunk];
      float zz[kMergeChunk];
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        if (s0 + k < NS) {
          const int si = s0 + k < ns_pair ? s0 + k : p.nsplit + (s0 + k - ns_pair);  // record index
          const float* rec = base_bh + si * REC;
          ml[k] = load_coherent2(rec + off_ml);
          av[k] = load_coherent2(rec + off_a);
          zz[k] = want_z ? load_coherent2(rec + off_ml + 2).x : 0.f;
        } else {
          ml[k] = make_float2(kNegInf, 0.f);
          av[k] = make_float2(0.f, 0.f);
          zz[k] = 0.f;
        }
      }
      float cm = kNegInf;
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) cm = fmaxf(cm, ml[k].x);
      const float Mn = fmaxf(M, cm);
      if (Mn == kNegInf) continue;
      const float sc = exp2_approx(M - Mn);  // 0 while M is still -inf
      L *= sc;
      Z *= sc;
      A0 *= sc;
      A1 *= sc;
#pragma unroll
      for (int k = 0; k < kMergeChunk; ++k) {
        const float f = ml[k].x == kNegInf ? 0.f : exp2_approx(ml[k].x - Mn);
        L = fmaf(f, ml[k].y, L);
        Z = fmaf(f, zz[k], Z);
        A0 = fmaf(f, av[k].x, A0);
        A1 = fmaf(f, av[k].y, A1);
      }
      M = Mn;
    }
    const int hq = h * G + g;
    const half2_t o = {static_cast<_Float16>(A0 / L), static_cast<_Float16>(A1 / L)};
    *reinterpret_cast<half2_t*>(&p.out[(static_cast<size_t>(b) * Hq + hq) * D + d]) = o;
    if (d == 0 && p.lse) p.lse[static_cast<size_t>(b) * Hq + hq] = (M + __builtin_log2f(L)) * kLn2;
    // entropy -sum p ln p = lse - E_p[z] (z the natural-log logits): in base-2 units M + log2 L - Z / L
    if (want_z) entropy[static_cast<size_t>(b) * Hq + hq] = (M + __builtin_log2f(L) - Z / L) * kLn2;
  }
  if (st) {
    __syncthreads();  // every output of the merge is written
    if (tid == 0) st[3] = __builtin_amdgcn_s_memrealtime();
  }
  if (tid == 0) {
    __hip_atomic_store(&p.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (CLAIM) __hip_atomic_store(&p.work[static_cast<size_t>(bh) * kClaimStride], 0u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (FUSED) {
    if (n_host >= 0) {
      // no workgroup of this launch reads seq_len: the kv-head 0 merge stores the new length
      if (h == 0 && tid == 0) __hip_atomic_store(&c.seq_len[b], n_host + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (tid == 0 &&
               __hip_atomic_fetch_add(&p.seq_counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                   static_cast<unsigned>(c.H - 1)) {
      // every workgroup of (b, h) has read seq_len[b] before this merge; the last of the H merges
      // of sequence b publishes the new length (and resets the counter)
      __hip_atomic_store(&c.seq_len[b], c.seq_len[b] + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.seq_counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Every argument the kernel uses is consumed at entry, so its scalar loads are issued together and
// waited for once.
__device__ __forceinline__ void consume_args(const DecodeParams& p) {
  asm volatile("" ::"s"(p.c.H), "s"(p.c.T), "s"(p.c.max_blocks), "s"(p.c.num_phys), "s"(p.c.hot), "s"(p.c.cold),
               "s"(p.c.scales), "s"(p.c.headers), "s"(p.c.seq_len), "s"(p.q), "s"(p.sel), "s"(p.k_sel),
               "s"(p.partials), "s"(p.counters), "s"(p.nsplit), "s"(p.nparts), "s"(p.units_per_split),
               "s"(p.wg_order), "s"(p.work), "s"(p.qscale));
}

// Grid (split, kv-head, sequence) in the plan's workgroup order (see wg_coord).
// Waves per SIMD the register budget is sized for: fp16 tiles hold twice the registers of 8-bit ones.
template <int G, int BITS>
constexpr int decode_waves() { return (G > 4 || BITS == 0) ? 2 : 4; }

// STATS: the variant that also carries the entropy statistic (launched only when the cache view
// asks for it, with a static plan); the others hold no register for it.
// A fused step's launch arguments carry the lengths before the append (DecodeParamsFused).
__device__ __forceinline__ const DecodeParams& params_of(const DecodeParams& p) { return p; }
__device__ __forceinline__ const DecodeParams& params_of(const DecodeParamsFused& p) { return p.p; }
__device__ __forceinline__ const int32_t* host_lens_of(const DecodeParams&) { return nullptr; }
__device__ __forceinline__ const int32_t* host_lens_of(const DecodeParamsFused& p) {
  return p.p.host_lens ? p.n0 : nullptr;
}

template <int D, int G, int BITS, int MODE, bool FUSED, bool CLAIM, bool STATS = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves<G, BITS>()))) void decode_kernel(
    typename std::conditional<FUSED, DecodeParamsFused, DecodeParams>::type po) {
  const DecodeParams& p = params_of(po);
  consume_args(p);
  decode_body<D, G, BITS, MODE, FUSED, CLAIM, STATS>(p, wg_coord(p.wg_order), host_lens_of(po));
}

// Batch plans: the same grid read in the host-built order of the table (see wg_coord_table); a kernel
// of its own, so the table does not enlarge the arguments of every other launch.
template <int D, int G, int BITS, bool FUSED, bool CLAIM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves<G, BITS>()))) void
decode_kernel_ordered(DecodeParamsOrdered po) {
  consume_args(po.p);
  decode_body<D, G, BITS, kModeDense, FUSED, CLAIM, false>(po.p, wg_coord_table(po.order),
                                                           FUSED && po.p.host_lens ? po.n0 : nullptr);
}

// The fused step's arguments: the parameters and, with p.host_lens, the host mirror's lengths.
inline DecodeParamsFused fused_args(const DecodeParams& p) {
  DecodeParamsFused f;
  f.p = p;
  std::memset(f.n0, 0, sizeof(f.n0));
  if (p.host_lens) std::memcpy(f.n0, p.n0_host, sizeof(int32_t) * static_cast<size_t>(p.c.B));
  return f;
}

template <typename K, typename P>
hipError_t launch_k(K kernel, dim3 grid, int block, const P& p, const LaunchCtx& ctx) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D, int G, int BITS>
hipError_t launch_dg(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order) {
  const dim3 grid(grid_parts(p), p.c.H, p.c.B);  // (split, kv-head, sequence)
  if (p.host_lens && (p.c.B > kFusedLenMax || !p.n0_host || !p.k_new)) return hipErrorInvalidValue;
  if (p.c.entropy) {  // statistics: static plans in plain order only
    if (order || p.work || p.wg_order != kOrderPlain) return hipErrorInvalidValue;
    if (p.k_new)
      return launch_k(decode_kernel<D, G, BITS, kModeDense, true, false, true>, grid, kThreads, fused_args(p), ctx);
    if (p.store_units_base)
      return launch_k(decode_kernel<D, G, BITS, kModeStore, false, false, true>, grid, kThreads, p, ctx);
    if (p.sel) return launch_k(decode_kernel<D, G, BITS, kModeGather, false, false, true>, grid, kThreads, p, ctx);
    return launch_k(decode_kernel<D, G, BITS, kModeDense, false, false, true>, grid, kThreads, p, ctx);
  }
  if (order && !p.sel) {
    if (p.order_groups < 1 || p.order_groups > kOrderTableMax) return hipErrorInvalidValue;
    const dim3 tgrid(p.c.H, p.order_groups);  // (kv-head, table group)
    DecodeParamsOrdered po;
    po.p = p;
    std::memcpy(po.order, order, sizeof(po.order));
    std::memset(po.n0, 0, sizeof(po.n0));
    if (p.host_lens) std::memcpy(po.n0, p.n0_host, sizeof(int32_t) * static_cast<size_t>(p.c.B));
    if (p.work)
      return p.k_new ? launch_k(decode_kernel_ordered<D, G, BITS, true, true>, tgrid, kThreads, po, ctx)
                     : launch_k(decode_kernel_ordered<D, G, BITS, false, true>, tgrid, kThreads, po, ctx);
    return p.k_new ? launch_k(decode_kernel_ordered<D, G, BITS, true, false>, tgrid, kThreads, po, ctx)
                   : launch_k(decode_kernel_ordered<D, G, BITS, false, false>, tgrid, kThreads, po, ctx);
  }
  if (p.k_new)
    return p.work ? launch_k(decode_kernel<D, G, BITS, kModeDense, true, true>, grid, kThreads, fused_args(p), ctx)
                  : launch_k(decode_kernel<D, G, BITS, kModeDense, true, false>, grid, kThreads, fused_args(p), ctx);
  if (p.store_units_base) return launch_k(decode_kernel<D, G, BITS, kModeStore, false, false>, grid, kThreads, p, ctx);
  if (p.sel) return launch_k(decode_kernel<D, G, BITS, kModeGather, false, false>, grid, kThreads, p, ctx);
  return p.work ? launch_k(decode_kernel<D, G, BITS, kModeDense, false, true>, grid, kThreads, p, ctx)
                : launch_k(decode_kernel<D, G, BITS, kModeDense, false, false>, grid, kThreads, p, ctx);
}

}  // namespace detail

// The decode launches of one (head_dim, group, cold-tile format) instance (explicitly instantiated by
// decode_inst.hip, one object per instance).
template <int D, int G, int BITS>
hipError_t launch_decode_dgb(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order) {
  return detail::launch_dg<D, G, BITS>(p, ctx, order);
}

}  // namespace hkv
