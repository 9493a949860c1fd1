// HySparse-style top-K token selection over the INT8 cold zone (gfx950).
//
// KV Cache reuse page, 2 (Spatial Gating Module at inference): score every
// past key against the current query by cosine, split the scores into
// 64-token windows, softmax inside each window, then take the global top-K;
// 2.1: the cosine is computed in FP32, and the selection has a fixed width
// max_K = 512 padded with a mask.
//
//   topk_score_kernel   one wave per cold block (window): lane t scores token
//                       t as the mean over the kv-head's G query heads of
//                       cos(q, code_t) (the block scale cancels in a cosine),
//                       then the wave does the window softmax and stores p.
//   topk_select_kernel  one 1024-thread workgroup per (sequence, kv-head):
//                       4-pass 8-bit radix select of the K-th largest p (as
//                       fp32 bit patterns, order-preserving for p >= 0), then
//                       an index-ordered block-scan compaction that takes
//                       every p above the threshold and the lowest-index ties,
//                       so the output is ascending and deterministic.
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr float kNegInfT = -__builtin_inff();
constexpr int kSelThreads = 1024;

template <int D, int G>
__global__ __launch_bounds__(kThreads) void topk_score_kernel(TopkParams p) {
  constexpr int S = kBlockSize;
  __shared__ float qs[G][D];
  __shared__ float qn[G];
  const CacheView& c = p.c;
  const int H = c.H;
  const int split = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;
  const int h = bh % H;
  const int b = bh / H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const _Float16* qg = p.q + (static_cast<size_t>(b) * H * G + static_cast<size_t>(h) * G) * D;
  for (int i = tid; i < G * D; i += kThreads) qs[i / D][i % D] = static_cast<float>(qg[i]);
  __syncthreads();
  if (w < G) {  // query norms (fp32)
    float s2 = 0.f;
    for (int d = lane; d < D; d += 64) s2 = fmaf(qs[w][d], qs[w][d], s2);
    s2 = wave_sum(s2);
    if (lane == 0) qn[w] = __builtin_sqrtf(s2);
  }
  for (int g = kWaves + w; g < G; g += kWaves) {  // G > 4
    float s2 = 0.f;
    for (int d = lane; d < D; d += 64) s2 = fmaf(qs[g][d], qs[g][d], s2);
    s2 = wave_sum(s2);
    if (lane == 0) qn[g] = __builtin_sqrtf(s2);
  }
  __syncthreads();

  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  const size_t cap = static_cast<size_t>(c.max_blocks) * S;
  float* prob = p.prob + static_cast<size_t>(bh) * cap;
  const int C = p.units_per_split;
  for (int run = split; run * C < sg.n_blk; run += p.nsplit) {
    const int u_end = min(sg.n_blk, (run + 1) * C);
    for (int j = run * C + w; j < u_end; j += kWaves) {
      if (j >= c.max_blocks) continue;
      const int phys = c.headers[static_cast<size_t>(b) * c.max_blocks + j].phys_block;
      if (phys < 0 || phys >= c.num_phys) continue;
      const int nv = min(S, sg.n_cold - j * S);
      const uint4* tk = reinterpret_cast<const uint4*>(c.cold + tile_offset(phys, h, 0, H, S, D));
      asm volatile("" ::: "memory");  // re-read q from LDS per block instead of pinning G x D VGPRs
      float dot[G];
#pragma unroll
      for (int g = 0; g < G; ++g) dot[g] = 0.f;
      int n2 = 0;
#pragma unroll
      for (int ch = 0; ch < D / 16; ++ch) {
        const uint4 kw = tk[ch * S + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wd = word_of(kw, i);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int code = static_cast<int8_t>(static_cast<uint8_t>(wd >> (8 * k)));
            const float kf = static_cast<float>(code);
            n2 += code * code;  // exact integer |code|^2
#pragma unroll
            for (int g = 0; g < G; ++g) dot[g] = fmaf(qs[g][ch * 16 + i * 4 + k], kf, dot[g]);
          }
        }
      }
      const float kn = __builtin_sqrtf(static_cast<float>(n2));
      float csum = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float den = qn[g] * kn;
        csum += den > 0.f ? dot[g] / den : 0.f;
      }
      const bool valid = lane < nv;
      const float cs = valid ? csum / static_cast<float>(G) : kNegInfT;
      // softmax inside the window (= this block's valid tokens)
      const float mx = wave_max(cs);
      const float e = valid ? exp2_approx((cs - mx) * kLog2e) : 0.f;
      const float es = wave_sum(e);
      if (valid) prob[static_cast<size_t>(j) * S + lane] = e / es;
    }
  }
}

// Inclusive scan of v over the 1024-thread block; returns the exclusive prefix
// and writes the block total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < kSelThreads / 64; ++i) {
      const int s = wsum[i];
      wsum[i] = run;
      run += s;
    }
    wsum[kSelThreads / 64] = run;
  }
  __syncthreads();
  const int excl = wsum[w] + x - v;
  *total = wsum[kSelThreads / 64];
  __syncthreads();  // wsum is reused by the next scan
  return excl;
}

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkParams p) {
  constexpr int S = kBlockSize;
  __shared__ unsigned hist[256];
  __shared__ int wsum[kSelThreads / 64 + 1];
  __shared__ unsigned s_prefix, s_krem;
  const CacheView& c = p.c;
  const int bh = blockIdx.x;
  const int b = bh / c.H;
  const int tid = threadIdx.x;
  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  const int n = min(sg.n_cold, c.max_blocks * S);  // never read past this (sequence, head)'s row
  const int K = p.k;
  int32_t* out = p.out_idx + static_cast<size_t>(bh) * K;
  const size_t cap = static_cast<size_t>(c.max_blocks) * S;
  const unsigned* keys = reinterpret_cast<const unsigned*>(p.prob + static_cast<size_t>(bh) * cap);

  if (n <= K) {
    for (int i = tid; i < K; i += kSelThreads) out[i] = i < n ? i : -1;
    return;
  }
  // ---- radix select: the K-th largest key and how many copies of it to take
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const unsigned key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      unsigned cum = 0;
      int dgt = 255;
      for (; dgt > 0; --dgt) {
        if (cum + hist[dgt] >= krem) break;
        cum += hist[dgt];
      }
      s_prefix = prefix | (static_cast<unsigned>(dgt) << shift);
      s_krem = krem - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
    __syncthreads();
  }
  const unsigned tau = prefix;
  const int need_eq = static_cast<int>(krem);
  // ---- ordered compaction in token order
  int carry_sel = 0, carry_eq = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + tid;
    const unsigned key = i < n ? keys[i] : 0u;
    const int is_eq = (i < n && key == tau) ? 1 : 0;
    const int is_gt = (i < n && key > tau) ? 1 : 0;
    int eq_total;
    const int eq_excl = block_exclusive_scan(is_eq, wsum, &eq_total);
    const int take = (is_gt || (is_eq && carry_eq + eq_excl < need_eq)) ? 1 : 0;
    int sel_total;
    const int sel_excl = block_exclusive_scan(take, wsum, &sel_total);
    if (take && carry_sel + sel_excl < K) out[carry_sel + sel_excl] = i;
    carry_eq += eq_total;
    carry_sel += sel_total;
  }
}

template <typename Kf>
hipError_t launch_t(Kf kernel, int grid, int block, const TopkParams& p, const LaunchCtx& ctx) {
  if (grid <= 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t launch_tg(const TopkParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  hipError_t e = launch_t(topk_score_kernel<D, G>, p.c.B * p.c.H * p.nsplit, kThreads, p, a);
  if (e != hipSuccess) return e;
  return launch_t(topk_select_kernel, p.c.B * p.c.H, kSelThreads, p, b);
}

template <int D>
hipError_t launch_td(const TopkParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  switch (p.G) {
    case 1: return launch_tg<D, 1>(p, a, b);
    case 2: return launch_tg<D, 2>(p, a, b);
    case 4: return launch_tg<D, 4>(p, a, b);
    case 8: return launch_tg<D, 8>(p, a, b);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

using namespace detail;

hipError_t launch_topk(const TopkParams& p, const LaunchCtx& score_ctx, const LaunchCtx& sel_ctx) {
  return p.c.D == 128 ? launch_td<128>(p, score_ctx, sel_ctx) : launch_td<64>(p, score_ctx, sel_ctx);
}

}  // namespace hkv
