// Split-K decode attention over the hybrid cache, and its log-sum-exp combine
// (gfx950, wave64).
//
// out[b][hq] = softmax(q . K^T / sqrt(d)) . V over the FP16 hot zone and the
// dequantised INT8 cold blocks (Hybrid KV Cache page 2.1 and 4.2: hot part in
// full precision, cold blocks dequantised on read; here one joint softmax).
//
// Work decomposition.  For each (sequence, kv-head) the attended tokens are
// split into "units": unit 0 is the hot zone (when non-empty), unit 1+j is
// cold block j (dense mode) or the j-th run of 64 selected cold tokens
// (sparse mode, KV Cache reuse page 2: only the selected tokens are loaded).
// A workgroup of 4 waves owns one split = a run of units_per_split units
// (round-robin over runs when a sequence has more units than the grid
// covers), each wave streams every 4th unit, keeps an fp32 online softmax
// (m, l, acc) for the G query heads of the kv-head, and the 4 waves are merged
// in LDS into one partial.  decode_combine merges the partials of all splits.
//
// Cold tiles are laid out so that one 16-byte load per lane is coalesced and
// lands exactly the bytes a lane needs: lane t gets 16 channels of token t
// from a K tile, lane l gets 16 tokens of channel l from a V tile.  Codes are
// converted to fp32 in registers; the block scale is applied once per block
// (to the logits for K, to the block's accumulated p.v for V).
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr float kNegInf = -__builtin_inff();

template <int D, int G>
struct WaveState {
  static constexpr int NDL = D / 64;  // channels owned per lane in p.v
  float m[G];                         // running max of base-2 logits
  float l[G];                         // lane-partial sum of p (reduced at the end)
  float acc[G][NDL];                  // acc[g][i] for channel lane + 64 i
};

template <int D, int G>
struct DecodeSmem {
  float q[G][D];                      // query rows, fp32
  float pw[kWaves][64][G];            // per-wave softmax weights of the current unit
  float wm[kWaves][G];
  float wl[kWaves][G];
  float wacc[kWaves][G][D];
};

// Online-softmax update shared by every unit type: z[g] are this lane's
// base-2 logits (-inf for masked lanes).  Returns the rescale factor alpha[g]
// and leaves the weights p in pw[lane][g].
template <int D, int G>
__device__ __forceinline__ void softmax_step(WaveState<D, G>& st, const float (&z)[G], float (&alpha)[G],
                                             float (*pw)[G], int lane) {
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mb = wave_max(z[g]);
    const float mn = fmaxf(st.m[g], mb);
    // a unit whose lanes are all masked (sparse padding) leaves the state unchanged
    const bool none = mn == kNegInf;
    alpha[g] = none ? 1.f : exp2_approx(st.m[g] - mn);  // 0 when the old max is -inf
    const float pg = none ? 0.f : exp2_approx(z[g] - mn);
    st.l[g] = st.l[g] * alpha[g] + pg;
    st.m[g] = mn;
    pw[lane][g] = pg;
  }
  wave_lds_sync();
}

// ---- hot zone unit: FP16 rows of the ring, slots [0, n_hot)
template <int D, int G>
__device__ void hot_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const _Float16* hot_bh, int n_hot, float qscale,
                         int w, int lane) {
  constexpr int NDL = D / 64;
  for (int base = 0; base < n_hot; base += 64) {
    const int slot = base + lane;
    const bool valid = slot < n_hot;
    float z[G];
#pragma unroll
    for (int g = 0; g < G; ++g) z[g] = 0.f;
    asm volatile("" ::: "memory");
    if (valid) {
      const uint4* krow = reinterpret_cast<const uint4*>(hot_bh + static_cast<size_t>(slot) * 2 * D);
#pragma unroll
      for (int v = 0; v < D / 8; ++v) {
        const uint4 kw = krow[v];
        float kf[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kf[2 * i] = half_lo(word_of(kw, i));
          kf[2 * i + 1] = half_hi(word_of(kw, i));
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int i = 0; i < 8; ++i) z[g] = fmaf(sm.q[g][v * 8 + i], kf[i], z[g]);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) z[g] = valid ? z[g] * qscale : kNegInf;
    float alpha[G];
    softmax_step<D, G>(st, z, alpha, sm.pw[w], lane);
    float accb[G][NDL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NDL; ++i) accb[g][i] = 0.f;
    const int cnt = min(64, n_hot - base);
    for (int t = 0; t < cnt; ++t) {
      const _Float16* vrow = hot_bh + (static_cast<size_t>(base + t) * 2 + 1) * D;
      float vv[NDL];
#pragma unroll
      for (int i = 0; i < NDL; ++i) vv[i] = static_cast<float>(vrow[lane + 64 * i]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pg = sm.pw[w][t][g];
#pragma unroll
        for (int i = 0; i < NDL; ++i) accb[g][i] = fmaf(pg, vv[i], accb[g][i]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NDL; ++i) st.acc[g][i] = st.acc[g][i] * alpha[g] + accb[g][i];
    wave_lds_sync();  // pw is rewritten by the next unit
  }
}

// ---- logits of one lane's K row: lane holds D/16 16-byte chunks of int8 codes
template <int D, int G>
__device__ __forceinline__ void k_row_dot(const uint4 (&kr)[D / 16], const DecodeSmem<D, G>& sm, float (&z)[G]) {
  // Re-read the query from LDS for every unit: keeping G x D floats live in
  // VGPRs across the unit loop would cut occupancy to one wave per SIMD.
  asm volatile("" ::: "memory");
#pragma unroll
  for (int g = 0; g < G; ++g) z[g] = 0.f;
#pragma unroll
  for (int ch = 0; ch < D / 16; ++ch) {
    float kf[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t wd = word_of(kr[ch], i);
#pragma unroll
      for (int k = 0; k < 4; ++k) kf[4 * i + k] = sbyte(wd, k);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) z[g] = fmaf(sm.q[g][ch * 16 + i], kf[i], z[g]);
  }
}

// ---- dense cold block unit
template <int D, int G>
__device__ void cold_block_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, int b, int h, int j,
                                int n_cold, float qscale, int w, int lane) {
  constexpr int S = kBlockSize;
  constexpr int NDL = D / 64;
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
  uint4 vr[NDL][S / 16];
#pragma unroll
  for (int i = 0; i < NDL; ++i)
#pragma unroll
    for (int tc = 0; tc < S / 16; ++tc) vr[i][tc] = tv[tc * D + lane + 64 * i];

  float z[G];
  k_row_dot<D, G>(kr, sm, z);
  const float zs = sK * qscale;
#pragma unroll
  for (int g = 0; g < G; ++g) z[g] = lane < nv ? z[g] * zs : kNegInf;
  float alpha[G];
  softmax_step<D, G>(st, z, alpha, sm.pw[w], lane);

  float accb[G][NDL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NDL; ++i) accb[g][i] = 0.f;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    float vv[NDL];
#pragma unroll
    for (int i = 0; i < NDL; ++i) vv[i] = sbyte(word_of(vr[i][t / 16], (t % 16) / 4), t % 4);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pg = sm.pw[w][t][g];
#pragma unroll
      for (int i = 0; i < NDL; ++i) accb[g][i] = fmaf(pg, vv[i], accb[g][i]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NDL; ++i) st.acc[g][i] = st.acc[g][i] * alpha[g] + accb[g][i] * sV;
  wave_lds_sync();
}

// ---- sparse unit: up to 64 selected cold tokens, gathered one row per lane
template <int D, int G>
__device__ void gather_unit(WaveState<D, G>& st, DecodeSmem<D, G>& sm, const CacheView& c, const int32_t* sel_bh,
                            int k_sel, int b, int h, int chunk, int n_cold, float qscale, int w, int lane) {
  constexpr int S = kBlockSize;
  constexpr int NDL = D / 64;
  const int e = chunk * 64 + lane;
  int idx = e < k_sel ? sel_bh[e] : -1;
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
  float z[G];
  k_row_dot<D, G>(kr, sm, z);
  const float zs = sK * qscale;
#pragma unroll
  for (int g = 0; g < G; ++g) z[g] = valid ? z[g] * zs : kNegInf;
  float alpha[G];
  softmax_step<D, G>(st, z, alpha, sm.pw[w], lane);
  // fold the per-token V scale into the weight; record where the token's V bytes live
#pragma unroll
  for (int g = 0; g < G; ++g) sm.pw[w][lane][g] *= sV;
  wave_lds_sync();

  float accb[G][NDL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NDL; ++i) accb[g][i] = 0.f;
  const int cnt = min(64, k_sel - chunk * 64);
  for (int i2 = 0; i2 < cnt; ++i2) {
    // token i2 of this run (uniform across the wave)
    const int idx2 = sel_bh[chunk * 64 + i2];
    if (idx2 < 0 || idx2 >= n_cold) continue;
    const int j2 = idx2 / S;
    if (j2 >= c.max_blocks) continue;
    const int phys2 = c.headers[static_cast<size_t>(b) * c.max_blocks + j2].phys_block;
    if (phys2 < 0 || phys2 >= c.num_phys) continue;
    const int t2 = idx2 % S;
    const int8_t* vt = c.cold + tile_offset(phys2, h, 1, c.H, S, D) + (t2 / 16) * D * 16 + (t2 % 16);
    float vv[NDL];
#pragma unroll
    for (int i = 0; i < NDL; ++i) vv[i] = static_cast<float>(vt[(lane + 64 * i) * 16]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float pg = sm.pw[w][i2][g];
#pragma unroll
      for (int i = 0; i < NDL; ++i) accb[g][i] = fmaf(pg, vv[i], accb[g][i]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < NDL; ++i) st.acc[g][i] = st.acc[g][i] * alpha[g] + accb[g][i];
  wave_lds_sync();
}

template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeParams p) {
  constexpr int S = kBlockSize;
  constexpr int NDL = D / 64;
  __shared__ DecodeSmem<D, G> sm;
  const CacheView& c = p.c;
  const int H = c.H;
  const int split = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;

  // query rows of this kv-head's group, fp32 in LDS
  const _Float16* qg = p.q + (static_cast<size_t>(b) * H * G + static_cast<size_t>(h) * G) * D;
  for (int i = tid; i < G * D; i += kThreads) sm.q[i / D][i % D] = static_cast<float>(qg[i]);
  __syncthreads();

  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  const int has_hot = sg.n_hot > 0 ? 1 : 0;
  const int n_cold_units = SPARSE ? cdiv(p.k_sel, 64) : sg.n_blk;
  const int units = has_hot + (sg.n_cold > 0 ? n_cold_units : 0);
  const _Float16* hot_bh = c.hot + (static_cast<size_t>(b) * H + h) * c.T * 2 * D;
  const int32_t* sel_bh = SPARSE ? p.sel + (static_cast<size_t>(b) * H + h) * p.k_sel : nullptr;

  WaveState<D, G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = kNegInf;
    st.l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < NDL; ++i) st.acc[g][i] = 0.f;
  }
  const int C = p.units_per_split;
  for (int run = split; run * C < units; run += p.nsplit) {
    const int u_end = min(units, (run + 1) * C);
    for (int u = run * C + w; u < u_end; u += kWaves) {
      if (u < has_hot) {
        hot_unit<D, G>(st, sm, hot_bh, sg.n_hot, p.qscale, w, lane);
      } else if (SPARSE) {
        gather_unit<D, G>(st, sm, c, sel_bh, p.k_sel, b, h, u - has_hot, sg.n_cold, p.qscale, w, lane);
      } else {
        cold_block_unit<D, G>(st, sm, c, b, h, u - has_hot, sg.n_cold, p.qscale, w, lane);
      }
    }
  }
  // ---- merge the 4 waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float lsum = wave_sum(st.l[g]);
    if (lane == 0) {
      sm.wm[w][g] = st.m[g];
      sm.wl[w][g] = lsum;
    }
#pragma unroll
    for (int i = 0; i < NDL; ++i) sm.wacc[w][g][lane + 64 * i] = st.acc[g][i];
  }
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

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
  const int Hq = p.c.H * p.G;
  const int b = blockIdx.x / Hq;
  const int hq = blockIdx.x % Hq;
  const int h = hq / p.G, g = hq % p.G;
  const int d = threadIdx.x;
  const size_t stride = static_cast<size_t>(p.G) * (D + 2);
  const float* base = p.partials + ((static_cast<size_t>(b) * p.c.H + h) * p.nsplit) * stride + g * (D + 2);
  float M = kNegInf;
  for (int s = 0; s < p.nsplit; ++s) M = fmaxf(M, base[s * stride]);
  float L = 0.f, A = 0.f;
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
  return launch_k(decode_combine_kernel<D>, p.c.B * p.c.H * p.G, D, p, comb_ctx);
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
