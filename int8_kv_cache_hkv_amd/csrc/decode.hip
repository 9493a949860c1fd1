// Split-K decode attention over the hybrid cache, and its log-sum-exp combine
// (gfx950, wave64, MFMA).
//
// out[b][hq] = softmax(q . K^T / sqrt(d)) . V over the FP16 hot zone and the
// dequantised INT8 cold blocks (Hybrid KV Cache page 2.1 and 4.2: hot part in
// full precision, cold blocks dequantised on read; here one joint softmax).
//
// Work decomposition.  For each (sequence, kv-head) the cold tokens are split
// into "units": unit j is cold block j (dense mode) or the j-th run of 64
// selected cold tokens (sparse mode, KV Cache reuse page 2: only the selected
// tokens are loaded).  The FP16 hot zone is attended by decode_combine.
// A workgroup of 4 waves owns one split = a run of units_per_split units
// (round-robin over runs when a sequence has more units than the grid
// covers); each wave streams every 4th unit of the run and keeps an fp32
// online softmax (m, l, acc) for the G query heads of the kv-head; the 4
// waves are merged in LDS into one partial per split, and decode_combine
// attends the hot zone and merges it with the splits.
//
// Per unit of 64 tokens a wave does:
//   QK  v_mfma_f32_4x4x4f16: B operand = 4 channels of the lane's own token
//       (lane = token), A operand = 4 channels of query row lane%4 (from LDS),
//       so lane t ends with the logits of token t for 4 query heads.  INT8
//       codes become exact fp16 values with a byte permute + packed subtract.
//   PV  v_mfma_f32_4x4x1f32 (fp32 inputs, no rounding of p): B operand = the
//       value code of token t at the lane's channel, A operand = p of token t
//       for query row lane%4 (from LDS, with the block's V scale folded in), so
//       lane c accumulates out[g][c] for 4 query heads.
// Cold tiles are laid out so that one coalesced 16-byte load per lane lands
// exactly these operands: lane t gets 16 channels of token t from a K tile,
// lane c gets 16 tokens of channel c from a V tile.
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr float kNegInf = -__builtin_inff();
constexpr int kHotChunk = 32;         // hot-zone slots staged through LDS at a time

template <int D, int G>
struct Cfg {
  static constexpr int NQ = (G + 3) / 4;   // groups of 4 query heads (MFMA rows)
  static constexpr int NDL = D / 64;       // channel passes of 64 lanes
  static constexpr int QROW = D + 8;       // padded fp16 query row in LDS (spreads the 4 rows over banks)
  static constexpr int PROW = 64 + 4;      // padded fp32 weight row in LDS
};

template <int D, int G>
struct DecodeSmem {
  using C = Cfg<D, G>;
  _Float16 qh[C::NQ][4][C::QROW];          // query rows (fp16, exact), zero rows past G
  float pw[kWaves][C::NQ][4][C::PROW];     // per-wave weights p[g][token] of the current unit
  float wm[kWaves][4 * C::NQ];
  float wl[kWaves][4 * C::NQ];
  float wacc[kWaves][4 * C::NQ][D];
  long long voff[kWaves][64];              // sparse mode: byte offset of each selected token's V column
};

template <int D, int G>
struct HotSmem {
  using C = Cfg<D, G>;
  _Float16 qh[C::NQ][4][C::QROW];          // query rows (fp16), zero rows past G
  float acc[G][D];
  float z[4 * C::NQ][kHotChunk];           // softmax weights of the current chunk (rows stay 0 past cnt)
  float m[4 * C::NQ], l[4 * C::NQ], alpha[4 * C::NQ];
  _Float16 kv[kHotChunk * (2 * D + 8)];     // staged [K|V] rows of the current chunk (padded)
};

template <int D, int G>
struct WaveState {
  using C = Cfg<D, G>;
  float m[4 * C::NQ];                      // running max of base-2 logits (wave-uniform)
  float l[4 * C::NQ];                      // lane-partial sum of p
  float4_t acc[C::NQ][C::NDL][2];          // [quad][pass][token parity]: out[4quad + r][64 pass + lane]
};

template <int D, int G>
__device__ __forceinline__ half4_t q_operand(const DecodeSmem<D, G>& sm, int quad, int lane, int k0) {
  return *reinterpret_cast<const half4_t*>(&sm.qh[quad][lane & 3][k0]);
}

// Online-softmax update for one unit: s[quad][r] are this lane's raw logits for
// query rows 4quad + r; `scale` turns them into base-2 logits; masked lanes give
// p = 0.  Leaves p * vscale in pw (PV operand), rescales the accumulators.
template <int D, int G>
__device__ __forceinline__ void softmax_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const float4_t (&s)[Cfg<D, G>::NQ],
                                             bool valid, float scale, float vscale, int w, int lane) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * quad + r;
      const float z = valid ? s[quad][r] * scale : kNegInf;
      const float mb = wave_max_dpp(z);
      const float mn = fmaxf(st.m[g], mb);
      const bool none = mn == kNegInf;  // all lanes masked (sparse padding): state unchanged
      const float alpha = none ? 1.f : exp2_approx(st.m[g] - mn);
      const float p = none ? 0.f : exp2_approx(z - mn);
      st.l[g] = st.l[g] * alpha + p;
      st.m[g] = mn;
      sm.pw[w][quad][r][lane] = p * vscale;
#pragma unroll
      for (int ps = 0; ps < C::NDL; ++ps) {
        st.acc[quad][ps][0][r] *= alpha;
        st.acc[quad][ps][1][r] *= alpha;
      }
    }
  }
  wave_lds_sync();
}

// PV over the 64 tokens of a unit whose value codes are lane-resident:
// vr[pass][tc] holds tokens 16tc..16tc+15 of channel 64 pass + lane.
template <int D, int G>
__device__ __forceinline__ void pv_codes(WaveState<D, G>& st, const DecodeSmem<D, G>& sm, const uint4 (&vr)[Cfg<D, G>::NDL][4],
                                         int w, int lane) {
  using C = Cfg<D, G>;
#pragma unroll
  for (int t0 = 0; t0 < 64; t0 += 4) {
    asm volatile("" ::: "memory");  // convert codes 4 tokens at a time (bounds live VGPRs)
    float4_t pa[C::NQ];
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad) pa[quad] = *reinterpret_cast<const float4_t*>(&sm.pw[w][quad][lane & 3][t0]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = t0 + k;
#pragma unroll
      for (int ps = 0; ps < C::NDL; ++ps) {
        const float vf = sbyte(word_of(vr[ps][t / 16], (t % 16) / 4), t % 4);
#pragma unroll
        for (int quad = 0; quad < C::NQ; ++quad) st.acc[quad][ps][t & 1] = mfma_pv(pa[quad][k], vf, st.acc[quad][ps][t & 1]);
      }
    }
  }
}

// ---------------------------------------------------------------- units
// Logits of the lane's K row (D/16 chunks of 16 int8 codes) for every query row.
template <int D, int G>
__device__ __forceinline__ void qk_codes(const uint4 (&kr)[D / 16], const DecodeSmem<D, G>& sm, int lane,
                                         float4_t (&s)[Cfg<D, G>::NQ]) {
  using C = Cfg<D, G>;
  asm volatile("" ::: "memory");  // re-read the query operand from LDS for every unit
  float4_t s2[C::NQ];  // second accumulator chain: halves the dependent MFMA chain
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] = s2[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) {
    asm volatile("" ::: "memory");  // bound how far the query-operand LDS reads are hoisted
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const half4_t b = codes_to_half4(word_of(kr[ch], wd));
      const int k0 = ch * 16 + wd * 4;
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) {
        if (wd & 1) s2[quad] = mfma_qk(q_operand(sm, quad, lane, k0), b, s2[quad]);
        else s[quad] = mfma_qk(q_operand(sm, quad, lane, k0), b, s[quad]);
      }
    }
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] += s2[quad];
}

// Dense cold block j.
template <int D, int G>
__device__ void cold_block_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, int b, int h, int j,
                                int phys_hint, int n_cold, float qscale, int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  if (j >= c.max_blocks) return;
  // phys_hint: the header already read for this block (-2: not read yet)
  const int phys = phys_hint != -2 ? phys_hint : c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
  if (phys < 0 || phys >= c.num_phys) return;
  const int nv = min(S, n_cold - j * S);
  const float sK = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 0];
  const float sV = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 1];
  const uint4* tk = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 0, c.H, S, D));
  const uint4* tv = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 1, c.H, S, D));
  uint4 kr[D / 16];
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) kr[ch] = load_stream(tk + ch * S + lane);
  uint4 vr[C::NDL][4];
#pragma unroll
  for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) vr[ps][tc] = load_stream(tv + tc * D + 64 * ps + lane);
  float4_t s[C::NQ];
  qk_codes<D, G>(kr, sm, lane, s);
  softmax_unit<D, G>(st, sm, s, lane < nv, sK * qscale, sV, w, lane);
  pv_codes<D, G>(st, sm, vr, w, lane);
  wave_lds_sync();
}

// Sparse unit: up to 64 selected cold tokens, one gathered row per lane.  For
// PV, lane c needs the value code of every selected token at channel c: the
// tokens' V-tile offsets go through LDS and the byte loads of 16 tokens are
// issued together, so the unit pays four memory latencies, not 64.
template <int D, int G>
__device__ void gather_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, const int32_t* sel_bh,
                            int k_sel, int b, int h, int chunk, int n_cold, float qscale, int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  constexpr int TB = 16;  // tokens whose value bytes are loaded together
  const int e = chunk * 64 + lane;
  const int idx = e < k_sel ? sel_bh[e] : -1;
  int phys = -1;
  if (idx >= 0 && idx < n_cold) {
    const int j = idx / S;
    if (j < c.max_blocks) phys = c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
  }
  const bool valid = phys >= 0 && phys < c.num_phys;
  const int t = valid ? idx % S : 0;
  float sK = 0.f, sV = 0.f;
  uint4 kr[D / 16];
  if (valid) {
    sK = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 0];
    sV = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 1];
    const uint4* tk = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 0, c.H, S, D));
#pragma unroll
    for (int ch = 0; ch < D / 16; ++ch) kr[ch] = tk[ch * S + t];
  } else {
#pragma unroll
    for (int ch = 0; ch < D / 16; ++ch) kr[ch] = make_uint4(0, 0, 0, 0);
  }
  // byte offset of (token, channel 0) in the cold pool, or -1 for a masked lane
  sm.voff[w][lane] = valid ? static_cast<long long>(tile_offset(phys, h, 1, c.H, S, D)) + (t / 16) * D * 16 + (t % 16)
                           : -1ll;
  float4_t s[C::NQ];
  qk_codes<D, G>(kr, sm, lane, s);
  softmax_unit<D, G>(st, sm, s, valid, sK * qscale, sV, w, lane);
  const int cnt = min(64, k_sel - chunk * 64);
  for (int tb = 0; tb < cnt; tb += TB) {
    float vf[TB][C::NDL];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const long long off = sm.voff[w][tb + k];  // uniform across the wave
#pragma unroll
      for (int ps = 0; ps < C::NDL; ++ps)
        vf[k][ps] = off >= 0 ? static_cast<float>(c.cold[off + (64 * ps + lane) * 16]) : 0.f;
    }
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += 4) {
      float4_t pa[C::NQ];
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad)
        pa[quad] = *reinterpret_cast<const float4_t*>(&sm.pw[w][quad][lane & 3][tb + t0]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
          for (int quad = 0; quad < C::NQ; ++quad)
            st.acc[quad][ps][k & 1] = mfma_pv(pa[quad][k], vf[t0 + k][ps], st.acc[quad][ps][k & 1]);
    }
  }
  wave_lds_sync();
}

// Partials are exchanged between workgroups that may sit on different XCDs
// (each with its own L2).  They are written and read with agent-scope relaxed
// atomic accesses (device-coherent sc1 loads/stores), so publishing them needs
// only a wait for the stores to complete, not an L2-wide writeback.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Partial record of one split: m (base-2 log units), l, acc[D] for each of the G query heads.
template <int D>
__device__ __forceinline__ float* partial_ptr(const DecodeParams& p, int bh, int split, int g) {
  return p.partials + ((static_cast<size_t>(bh) * (p.nsplit + 1) + split) * p.G + g) * (D + 2);
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

// ---- cold split: stream its units, merge the 4 waves, write the partial
template <int D, int G, bool SPARSE>
__device__ void cold_split(const DecodeParams& p, DecodeSmem<D, G>& sm, int b, int h, int bh, int split) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  constexpr int NG = 4 * C::NQ;
  const CacheView& c = p.c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  // issue the length and this wave's first header read together with the query copy
  const int n_seq = c.seq_len[b];
  const int u0 = split * p.units_per_split + w;
  const int phys0 = (!SPARSE && u0 < c.max_blocks) ? c.headers[static_cast<size_t>(b) * c.max_blocks + u0].phys_block : -1;
  copy_query<D, G>(p.q + (static_cast<size_t>(b) * c.H * G + static_cast<size_t>(h) * G) * D, sm.qh, tid);
  __syncthreads();

  const SeqGeom sg = seq_geom(n_seq, c.T, S);
  const int units = sg.n_cold > 0 ? (SPARSE ? cdiv(p.k_sel, 64) : sg.n_blk) : 0;
  const int32_t* sel_bh = SPARSE ? p.sel + static_cast<size_t>(bh) * p.k_sel : nullptr;

  WaveState<D, G> st;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    st.m[g] = kNegInf;
    st.l[g] = 0.f;
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps) st.acc[quad][ps][0] = st.acc[quad][ps][1] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int CU = p.units_per_split;
  for (int run = split; run * CU < units; run += p.nsplit) {
    const int u_end = min(units, (run + 1) * CU);
    for (int u = run * CU + w; u < u_end; u += kWaves) {
      if (SPARSE) {
        gather_unit<D, G>(st, sm, c, sel_bh, p.k_sel, b, h, u, sg.n_cold, p.qscale, w, lane);
      } else {
        cold_block_unit<D, G>(st, sm, c, b, h, u, u == u0 ? phys0 : -2, sg.n_cold, p.qscale, w, lane);
      }
    }
  }
  // merge the 4 waves: lane holds out[4quad + r][64 pass + lane]
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float lsum = wave_sum(st.l[g]);
    if (lane == 0) {
      sm.wm[w][g] = st.m[g];
      sm.wl[w][g] = lsum;
    }
  }
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad)
#pragma unroll
    for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.wacc[w][4 * quad + r][64 * ps + lane] = st.acc[quad][ps][0][r] + st.acc[quad][ps][1][r];
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int g = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.wm[ww][g]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if (sm.wm[ww][g] == kNegInf) continue;
        const float f = exp2_approx(sm.wm[ww][g] - M);
        L += f * sm.wl[ww][g];
        A += f * sm.wacc[ww][g][d];
      }
    }
    float* pg = partial_ptr<D>(p, bh, split, g);
    store_coherent(pg + 2 + d, A);
    if (d == 0) {
      store_coherent(pg, M);
      store_coherent(pg + 1, L);
    }
  }
}

// ---- hot split: the FP16 ring (Hybrid KV Cache page 2.1: the most recent
// tokens in full precision).  Chunks of kHotChunk slots are staged through LDS
// with coalesced loads; wave 0 computes the logits with the same MFMA as the
// cold blocks (lane = slot, fp16 K rows are already MFMA operands) and the
// softmax weights; all four waves then accumulate thread (g, d) = sum_t p v.
template <int D, int G>
__device__ void hot_split(const DecodeParams& p, HotSmem<D, G>& hm, int b, int h, int bh) {
  using C = Cfg<D, G>;
  constexpr int NG = 4 * C::NQ;
  constexpr int ROW = 2 * D + 8;          // padded fp16 [K|V] row
  constexpr int VPR = 2 * D / 8;          // 16-byte vectors per row
  const CacheView& c = p.c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n_seq = c.seq_len[b];
  copy_query<D, G>(p.q + (static_cast<size_t>(b) * c.H * G + static_cast<size_t>(h) * G) * D, hm.qh, tid);
  for (int i = tid; i < G * D; i += kThreads) hm.acc[i / D][i % D] = 0.f;
  const SeqGeom sg = seq_geom(n_seq, c.T, kBlockSize);
  const _Float16* hot_bh = c.hot + static_cast<size_t>(bh) * c.T * 2 * D;
  float m[NG], l[NG];  // wave 0's running softmax state (wave-uniform)
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
  }
  for (int base = 0; base < sg.n_hot; base += kHotChunk) {
    const int cnt = min(kHotChunk, sg.n_hot - base);
    const uint4* src = reinterpret_cast<const uint4*>(hot_bh + static_cast<size_t>(base) * 2 * D);
    constexpr int NV = (kHotChunk * VPR + kThreads - 1) / kThreads;
    uint4 buf[NV];  // all of the chunk's loads in flight together
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = tid + k * kThreads;
      buf[k] = i < cnt * VPR ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int i = tid + k * kThreads;
      if (i < kHotChunk * VPR) *reinterpret_cast<uint4*>(&hm.kv[(i / VPR) * ROW + (i % VPR) * 8]) = buf[k];
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
          s[quad] = mfma_qk(*reinterpret_cast<const half4_t*>(&hm.qh[quad][lane & 3][k0]), bk, s[quad]);
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
          m[g] = mn;
          if (lane < kHotChunk) hm.z[g][lane] = pt;
          if (lane == 0) hm.alpha[g] = alpha;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += kThreads) {
      const int g = i / D, d = i % D;
      float a = hm.acc[g][d] * hm.alpha[g];
      for (int t = 0; t < cnt; ++t) a = fmaf(hm.z[g][t], static_cast<float>(hm.kv[t * ROW + D + d]), a);  // rows past cnt are not staged
      hm.acc[g][d] = a;
    }
    __syncthreads();
  }
  if (w == 0 && lane == 0) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      hm.m[g] = m[g];
      hm.l[g] = l[g];
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float* pg = partial_ptr<D>(p, bh, p.nsplit, g);
    store_coherent(pg + 2 + d, hm.acc[g][d]);
    if (d == 0) {
      store_coherent(pg, hm.m[g]);
      store_coherent(pg + 1, hm.l[g]);
    }
  }
}

// One launch per decode call: B*H*(nsplit + 1) workgroups; for each (sequence,
// kv-head) nsplit cold splits and one hot split write partials, and the last
// of them to arrive merges all nsplit + 1 partials with the log-sum-exp rule
// (M = max m_s, L = sum e^(m_s - M) l_s, out = sum e^(m_s - M) acc_s / L) and
// writes the fp16 output.  Arrival is counted with a device-scope atomic in
// the workspace, which the merging workgroup resets to zero.
template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G > 4 ? 2 : 3))) void decode_kernel(DecodeParams p) {
  __shared__ union Smem {
    DecodeSmem<D, G> cold;
    HotSmem<D, G> hot;
  } sm;
  __shared__ int s_last;
  __shared__ float mw[kMaxSplits + 1][G];   // m_s, then e^(m_s - M)
  __shared__ float ml[kMaxSplits + 1][G];
  __shared__ float mM[G], mL[G];
  const CacheView& c = p.c;
  const int split = blockIdx.x % (p.nsplit + 1);
  const int bh = blockIdx.x / (p.nsplit + 1);
  const int h = bh % c.H;
  const int b = bh / c.H;
  const int tid = threadIdx.x;
  if (split < p.nsplit) {
    cold_split<D, G, SPARSE>(p, sm.cold, b, h, bh, split);
  } else {
    hot_split<D, G>(p, sm.hot, b, h, bh);
  }
  // ---- arrival: wait until this workgroup's partial stores are complete, count, and let the
  // last workgroup merge
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&p.counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<unsigned>(p.nsplit);
  __syncthreads();
  if (!s_last) return;
  // merge: (1) every m_s, l_s into LDS in one round and the weights e^(m_s - M);
  // (2) each thread's accumulator columns, 16 splits' loads in flight at a time
  const int NS = p.nsplit + 1;
  for (int i = tid; i < NS * G; i += kThreads) {
    const float* pg = partial_ptr<D>(p, bh, i / G, i % G);
    mw[i / G][i % G] = load_coherent(pg);
    ml[i / G][i % G] = load_coherent(pg + 1);
  }
  __syncthreads();
  for (int g = tid; g < G; g += kThreads) {
    float M = kNegInf;
    for (int s2 = 0; s2 < NS; ++s2) M = fmaxf(M, mw[s2][g]);
    float L = 0.f;
    for (int s2 = 0; s2 < NS; ++s2) {
      const float f = mw[s2][g] == kNegInf ? 0.f : exp2_approx(mw[s2][g] - M);
      mw[s2][g] = f;
      L = fmaf(f, ml[s2][g], L);
    }
    mM[g] = M;
    mL[g] = L;
  }
  __syncthreads();
  const int Hq = c.H * G;
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float A = 0.f;
    for (int s0 = 0; s0 < NS; s0 += 16) {
      float av[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) av[k] = s0 + k < NS ? load_coherent(partial_ptr<D>(p, bh, s0 + k, g) + 2 + d) : 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (s0 + k < NS) A = fmaf(mw[s0 + k][g], av[k], A);
    }
    const int hq = h * G + g;
    p.out[(static_cast<size_t>(b) * Hq + hq) * D + d] = static_cast<_Float16>(A / mL[g]);
    if (d == 0 && p.lse) p.lse[static_cast<size_t>(b) * Hq + hq] = (mM[g] + __builtin_log2f(mL[g])) * kLn2;
  }
  if (tid == 0) __hip_atomic_store(&p.counters[bh], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename K>
hipError_t launch_k(K kernel, int grid, int block, const DecodeParams& p, const LaunchCtx& ctx) {
  if (grid <= 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_dg(const DecodeParams& p, const LaunchCtx& ctx) {
  const int grid = p.c.B * p.c.H * (p.nsplit + 1);
  return p.sel ? launch_k(decode_kernel<D, G, true>, grid, kThreads, p, ctx)
               : launch_k(decode_kernel<D, G, false>, grid, kThreads, p, ctx);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, const LaunchCtx& a) {
  switch (p.G) {
    case 1: return launch_dg<D, 1>(p, a);
    case 2: return launch_dg<D, 2>(p, a);
    case 4: return launch_dg<D, 4>(p, a);
    case 8: return launch_dg<D, 8>(p, a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

using namespace detail;

hipError_t launch_decode(const DecodeParams& p, const LaunchCtx& ctx) {
  return p.c.D == 128 ? launch_d<128>(p, ctx) : launch_d<64>(p, ctx);
}

}  // namespace hkv
