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
constexpr int kCombineThreads = 128;  // >= head_dim and >= hot_tokens (both at most 128)

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
#pragma unroll
  for (int quad = 0; quad < C::NQ; ++quad) s[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) {
    asm volatile("" ::: "memory");  // bound how far the query-operand LDS reads are hoisted
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const half4_t b = codes_to_half4(word_of(kr[ch], wd));
      const int k0 = ch * 16 + wd * 4;
#pragma unroll
      for (int quad = 0; quad < C::NQ; ++quad) s[quad] = mfma_qk(q_operand(sm, quad, lane, k0), b, s[quad]);
    }
  }
}

// Dense cold block j.
template <int D, int G>
__device__ void cold_block_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, int b, int h, int j,
                                int n_cold, float qscale, int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  if (j >= c.max_blocks) return;
  const int phys = c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
  if (phys < 0 || phys >= c.num_phys) return;
  const int nv = min(S, n_cold - j * S);
  const float sK = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 0];
  const float sV = c.scales[(static_cast<size_t>(phys) * c.H + h) * 2 + 1];
  const uint4* tk = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 0, c.H, S, D));
  const uint4* tv = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 1, c.H, S, D));
  uint4 kr[D / 16];
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) kr[ch] = tk[ch * S + lane];
  uint4 vr[C::NDL][4];
#pragma unroll
  for (int ps = 0; ps < C::NDL; ++ps)
#pragma unroll
    for (int tc = 0; tc < 4; ++tc) vr[ps][tc] = tv[tc * D + 64 * ps + lane];
  float4_t s[C::NQ];
  qk_codes<D, G>(kr, sm, lane, s);
  softmax_unit<D, G>(st, sm, s, lane < nv, sK * qscale, sV, w, lane);
  pv_codes<D, G>(st, sm, vr, w, lane);
  wave_lds_sync();
}

// Sparse unit: up to 64 selected cold tokens, one gathered row per lane.
template <int D, int G>
__device__ void gather_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, const int32_t* sel_bh,
                            int k_sel, int b, int h, int chunk, int n_cold, float qscale, int w, int lane) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
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
  float4_t s[C::NQ];
  qk_codes<D, G>(kr, sm, lane, s);
  softmax_unit<D, G>(st, sm, s, valid, sK * qscale, sV, w, lane);
  const int cnt = min(64, k_sel - chunk * 64);
  for (int t0 = 0; t0 < cnt; t0 += 4) {
    float4_t pa[C::NQ];
#pragma unroll
    for (int quad = 0; quad < C::NQ; ++quad) pa[quad] = *reinterpret_cast<const float4_t*>(&sm.pw[w][quad][lane & 3][t0]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // token t0 + k of this run (uniform across the wave); a masked token has p = 0 and reads nothing
      const int i2 = t0 + k;
      const int idx2 = i2 < cnt ? sel_bh[chunk * 64 + i2] : -1;
      int phys2 = -1;
      if (idx2 >= 0 && idx2 < n_cold && idx2 / S < c.max_blocks)
        phys2 = c.headers[static_cast<size_t>(b) * c.max_blocks + idx2 / S].phys_block;
      const bool ok = phys2 >= 0 && phys2 < c.num_phys;
      const int8_t* vt = ok ? c.cold + tile_offset(phys2, h, 1, c.H, S, D) + ((idx2 % S) / 16) * D * 16 + (idx2 % 16)
                            : nullptr;
#pragma unroll
      for (int ps = 0; ps < C::NDL; ++ps) {
        const float vf = ok ? static_cast<float>(vt[(64 * ps + lane) * 16]) : 0.f;
#pragma unroll
        for (int quad = 0; quad < C::NQ; ++quad) st.acc[quad][ps][k & 1] = mfma_pv(pa[quad][k], vf, st.acc[quad][ps][k & 1]);
      }
    }
  }
  wave_lds_sync();
}

template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void decode_partial_kernel(DecodeParams p) {
  using C = Cfg<D, G>;
  constexpr int S = kBlockSize;
  constexpr int NG = 4 * C::NQ;
  __shared__ DecodeSmem<D, G> sm;
  const CacheView& c = p.c;
  const int H = c.H;
  const int split = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  // query rows of this kv-head's group as fp16 (exact copies), zero rows past G
  const _Float16* qg = p.q + (static_cast<size_t>(b) * H * G + static_cast<size_t>(h) * G) * D;
  for (int i = tid; i < NG * D; i += kThreads) {
    const int g = i / D, d = i % D;
    sm.qh[g / 4][g % 4][d] = g < G ? qg[g * D + d] : static_cast<_Float16>(0.f);
  }
  __syncthreads();

  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  const int units = sg.n_cold > 0 ? (SPARSE ? cdiv(p.k_sel, 64) : sg.n_blk) : 0;
  const int32_t* sel_bh = SPARSE ? p.sel + (static_cast<size_t>(b) * H + h) * p.k_sel : nullptr;

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
        cold_block_unit<D, G>(st, sm, c, b, h, u, sg.n_cold, p.qscale, w, lane);
      }
    }
  }
  // ---- merge the 4 waves: lane holds out[4quad + r][64 pass + lane]
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
  float* part = p.partials + (static_cast<size_t>(bh) * p.nsplit + split) * G * (D + 2);
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
    float* pg = part + g * (D + 2);
    pg[2 + d] = A;
    if (d == 0) {
      pg[0] = M;
      pg[1] = L;
    }
  }
}

// Hot zone + combine, one workgroup per (sequence, query head).  The FP16 hot
// zone (Hybrid KV Cache page 2.1: the most recent tokens in full precision) is
// attended here in fp32: thread t scores slot t, thread d accumulates channel
// d.  Its (m, l, acc) is then merged with the cold splits' partials by the
// log-sum-exp rule: M = max m_s, L = sum e^(m_s - M) l_s, out = sum e^(m_s - M)
// acc_s / L.
template <int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(DecodeParams p) {
  __shared__ float qf[D];
  __shared__ float ph[kCombineThreads];
  __shared__ float red[kCombineThreads / 64];
  const CacheView& c = p.c;
  const int Hq = c.H * p.G;
  const int b = blockIdx.x / Hq;
  const int hq = blockIdx.x % Hq;
  const int h = hq / p.G, g = hq % p.G;
  const int tid = threadIdx.x;
  for (int d = tid; d < D; d += kCombineThreads) qf[d] = static_cast<float>(p.q[(static_cast<size_t>(b) * Hq + hq) * D + d]);
  __syncthreads();
  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, kBlockSize);
  const _Float16* hot_bh = c.hot + (static_cast<size_t>(b) * c.H + h) * c.T * 2 * D;
  // ---- hot logits (base 2): slot t < n_hot (ring slots hold positions mod T; order is irrelevant)
  float z = kNegInf;
  if (tid < sg.n_hot) {
    const uint4* krow = reinterpret_cast<const uint4*>(hot_bh + static_cast<size_t>(tid) * 2 * D);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < D / 8; ++v) {
      const uint4 kw = krow[v];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wd = word_of(kw, i);
        acc = fmaf(qf[v * 8 + 2 * i], half_lo(wd), acc);
        acc = fmaf(qf[v * 8 + 2 * i + 1], half_hi(wd), acc);
      }
    }
    z = acc * p.qscale;
  }
  float mh = wave_max(z);
  if ((tid & 63) == 0) red[tid >> 6] = mh;
  __syncthreads();
  mh = red[0];
#pragma unroll
  for (int i = 1; i < kCombineThreads / 64; ++i) mh = fmaxf(mh, red[i]);
  __syncthreads();
  const float pt = tid < sg.n_hot ? exp2_approx(z - mh) : 0.f;
  ph[tid] = pt;
  float lh = wave_sum(pt);
  if ((tid & 63) == 0) red[tid >> 6] = lh;
  __syncthreads();
  lh = 0.f;
#pragma unroll
  for (int i = 0; i < kCombineThreads / 64; ++i) lh += red[i];
  // ---- merge with the cold partials
  const size_t stride = static_cast<size_t>(p.G) * (D + 2);
  const float* base = p.partials + ((static_cast<size_t>(b) * c.H + h) * p.nsplit) * stride + g * (D + 2);
  float M = mh;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, base[s * stride]);
  for (int d = tid; d < D; d += kCombineThreads) {
    float A = 0.f, L = 0.f;
    if (mh != kNegInf) {
      float ah = 0.f;
      for (int t = 0; t < sg.n_hot; ++t) ah = fmaf(ph[t], static_cast<float>(hot_bh[(static_cast<size_t>(t) * 2 + 1) * D + d]), ah);
      const float f = exp2_approx(mh - M);
      A = f * ah;
      L = f * lh;
    }
    for (int s = 0; s < p.nsplit; ++s) {
      const float ms = base[s * stride];
      if (ms == kNegInf) continue;
      const float f = exp2_approx(ms - M);
      L += f * base[s * stride + 1];
      A += f * base[s * stride + 2 + d];
    }
    p.out[(static_cast<size_t>(b) * Hq + hq) * D + d] = static_cast<_Float16>(A / L);
    if (d == 0 && p.lse) p.lse[static_cast<size_t>(b) * Hq + hq] = (M + __builtin_log2f(L)) * kLn2;
  }
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
hipError_t launch_dg(const DecodeParams& p, const LaunchCtx& part_ctx, const LaunchCtx& comb_ctx) {
  const int grid = p.c.B * p.c.H * p.nsplit;
  hipError_t e = p.sel ? launch_k(decode_partial_kernel<D, G, true>, grid, kThreads, p, part_ctx)
                       : launch_k(decode_partial_kernel<D, G, false>, grid, kThreads, p, part_ctx);
  if (e != hipSuccess) return e;
  return launch_k(decode_combine_kernel<D>, p.c.B * p.c.H * p.G, kCombineThreads, p, comb_ctx);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  switch (p.G) {
    case 1: return launch_dg<D, 1>(p, a, b);
    case 2: return launch_dg<D, 2>(p, a, b);
    case 4: return launch_dg<D, 4>(p, a, b);
    case 8: return launch_dg<D, 8>(p, a, b);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

using namespace detail;

hipError_t launch_decode(const DecodeParams& p, const LaunchCtx& part_ctx, const LaunchCtx& comb_ctx) {
  return p.c.D == 128 ? launch_d<128>(p, part_ctx, comb_ctx) : launch_d<64>(p, part_ctx, comb_ctx);
}

}  // namespace hkv
