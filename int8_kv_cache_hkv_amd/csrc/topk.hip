// HySparse-style top-K token selection over the INT8 cold zone (gfx950).
//
// KV Cache reuse page, 2 (Spatial Gating Module at inference): score every
// past key against the current query by cosine, split the scores into
// 64-token windows, softmax inside each window, then take the global top-K;
// 2.1: the cosine is computed in FP32, and the selection has a fixed width
// max_K = 512 padded with a mask.
//
//   topk_score_kernel   one wave per cold block (window), blocks streamed
//                       through a software pipeline: lane t scores token
//                       t as the mean over the kv-head's G query heads of
//                       cos(q, code_t) (the block scale cancels in a cosine);
//                       q.code comes from v_mfma_f32_4x4x4f16 on exact fp16
//                       copies (lane = token), |code|^2 from an integer dot4;
//                       then the wave does the window softmax and stores p.
//   topk_select_kernel  one 1024-thread workgroup per (sequence, kv-head):
//                       3-pass (11/10/10-bit) radix select of the K-th largest
//                       p (fp32 bit patterns, order-preserving for p >= 0) over
//                       lane-indexed histogram copies, restricted to keys at or
//                       above a floor taken from the per-thread maxima, then
//                       an index-ordered block-scan compaction that takes
//                       every p above the threshold and the lowest-index ties,
//                       so the output is ascending and deterministic.
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

constexpr float kNegInfT = -__builtin_inff();
// claim walk: units whose probabilities are staged in LDS before a write-out (each write-out drains
// the wave's loads; a wave walks about 16 units of the 32768-token workload, measured: stage of 16
// -> 91.8 us, 32 -> 90.0 us)
constexpr int kStage = 32;
constexpr int kSelThreads = 1024;

// Window probabilities of one cold block from its K tile: kr[ch] holds elements
// E ch .. E ch + E - 1 of the lane's token.  As each chunk is consumed its
// registers receive the same chunk of the next unit's K tile (rn; an empty
// descriptor when there is none), so the next tile streams in while this one
// is scored.
template <int D, int G, int BITS>
__device__ __forceinline__ float window_scores(uint4 (&kr)[D / Fmt<BITS>::kElems], const _Float16 (*qh)[4][D + 8],
                                               const float* qinv, int lane, int nv, __amdgpu_buffer_rsrc_t rn) {
  using F = Fmt<BITS>;
  constexpr int S = kBlockSize;
  constexpr int NQ = (G + 3) / 4;
  const uint32_t lo = static_cast<uint32_t>(lane) * 16u;
  // dot(q_g, k_t) for the lane's token t (MFMA, exact products) and |k_t|^2 (an integer dot4 of the
  // 8-bit codes; for 4-bit codes and fp16 values an fp32 dot2 of the exact fp16 operands)
  float4_t s[NQ];
#pragma unroll
  for (int quad = 0; quad < NQ; ++quad) s[quad] = float4_t{0.f, 0.f, 0.f, 0.f};
  int n2 = 0;
  float f2 = 0.f;
#pragma unroll
  for (int ch = 0; ch < D / F::kElems; ++ch) {
    asm volatile("" ::: "memory");  // keep the chunks in order: each refill is issued right after its use
    half4_t bk[F::kSteps];
#pragma unroll
    for (int st = 0; st < F::kSteps; ++st) {
      bk[st] = chunk_operand<BITS, false>(kr[ch], st);
      if constexpr (BITS == 8) {
        const uint32_t word = word_of(kr[ch], st);
        n2 = __builtin_amdgcn_sdot4(static_cast<int>(word), static_cast<int>(word), n2, false);
      } else {
        const half2_t a = {bk[st].x, bk[st].y}, b = {bk[st].z, bk[st].w};
        f2 = __builtin_amdgcn_fdot2(a, a, f2, false);
        f2 = __builtin_amdgcn_fdot2(b, b, f2, false);
      }
    }
    // every read of the chunk happens before the load that refills its registers: a read left
    // after it would need the old value in other registers, and the copy back at the end of the
    // walk's iteration would wait for every load in flight
#pragma unroll
    for (int st = 0; st < F::kSteps; ++st) asm volatile("" ::"v"(bk[st]) : "memory");
    asm volatile("" ::"v"(n2), "v"(f2) : "memory");
    kr[ch] = load_stream_buf(rn, lo + ch * S * 16);
#pragma unroll
    for (int st = 0; st < F::kSteps; ++st) {
      const int k0 = ch * F::kElems + st * 4;
#pragma unroll
      for (int quad = 0; quad < NQ; ++quad)
        s[quad] = mfma_qk(*reinterpret_cast<const half4_t*>(&qh[quad][lane & 3][k0]), bk[st], s[quad]);
    }
  }
  asm volatile("" ::: "memory");
  // c_t = mean over the G query heads of cos(q_g, k_t); cosine is scale-free, so codes suffice
  const float knorm2 = BITS == 8 ? static_cast<float>(n2) : f2;
  const float kinv = knorm2 > 0.f ? 1.f / __builtin_sqrtf(knorm2) : 0.f;
  float csum = 0.f;
#pragma unroll
  for (int quad = 0; quad < NQ; ++quad)
#pragma unroll
    for (int r = 0; r < 4; ++r) csum += s[quad][r] * qinv[4 * quad + r];
  const bool valid = lane < nv;
  const float cs = valid ? (csum * kinv) / static_cast<float>(G) : kNegInfT;
  // softmax inside the window (= this block's valid tokens)
  const float mx = wave_max_dpp(cs);
  const float e = valid ? exp2_approx((cs - mx) * kLog2e) : 0.f;
  const float es = wave_sum_dpp(e);
  return e / es;
}

// K tile of (phys, h) as a buffer resource (empty for phys < 0: loads read 0).
template <int D, int BITS>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_tile_rsrc(const CacheView& c, int phys, int h) {
  constexpr int TB = Fmt<BITS>::template tile_bytes<D>();
  const bool ok = phys >= 0;
  return make_rsrc(c.cold + tile_offset(ok ? phys : 0, h, 0, c.H, TB), ok ? TB : 0u);
}

// Grid (split, kv-head, sequence).  Each wave walks its cold blocks (the same
// walk as the decode's dense units); the first block's tile is requested with
// the query, each next one while the current one is scored.
template <int D, int G, int BITS, bool CLAIM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BITS == 0 ? 2 : 4))) void topk_score_kernel(
    TopkParams p) {
  constexpr int S = kBlockSize;
  constexpr int NQ = (G + 3) / 4;          // groups of 4 query heads (MFMA rows)
  constexpr int QROW = D + 8;              // padded fp16 query row
  constexpr int VPR = D / 8;               // 16-byte vectors per query row
  __shared__ _Float16 qh[NQ][4][QROW];
  __shared__ float qinv[4 * NQ];           // 1 / |q_g| (0 for a zero query or a padding row)
  __shared__ float pstage[CLAIM ? kWaves : 1][CLAIM ? kStage : 1][64];  // claim walk: staged window probabilities
  __shared__ int ustage[CLAIM ? kWaves : 1][CLAIM ? kStage : 1];
  asm volatile("" ::"s"(p.c.H), "s"(p.c.T), "s"(p.c.max_blocks), "s"(p.c.num_phys), "s"(p.c.cold),
               "s"(p.c.headers), "s"(p.c.seq_len), "s"(p.q), "s"(p.prob), "s"(p.nsplit), "s"(p.units_per_split),
               "s"(p.wg_order), "s"(p.work));
  const CacheView& c = p.c;
  const int H = c.H;
  const WgCoord wg = wg_coord(p.wg_order);
  const int split = wg.x, h = wg.y, b = wg.z;
  const int bh = b * H + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int CU = p.units_per_split;
  // first memory round: query rows, the length and this wave's header batch; then the first tile
  const _Float16* qg = p.q + (static_cast<size_t>(b) * H * G + static_cast<size_t>(h) * G) * D;
  const int qi = tid < 4 * NQ * VPR ? tid : 0;
  const bool q_ok = tid < G * VPR;
  const u32x4_t qv = reinterpret_cast<const u32x4_t*>(qg)[q_ok ? qi : 0];
  const int n_seq_lane = c.seq_len[opaque_index(b)];
  unsigned* work = CLAIM ? p.work + static_cast<size_t>(bh) * kClaimStride : nullptr;
  unsigned cl = 0;  // claim walk: the first claim travels with the first round
  int hb = CLAIM ? header_load(c, b, split * kWaves + w) : header_batch(c, b, 0, split, p.nsplit, CU, w, lane);
  if (CLAIM) cl = claim_issue(work, lane);
  int phys = CLAIM ? header_phys(c, hb) : __builtin_amdgcn_readlane(hb, 0);
  uint4 kr[D / Fmt<BITS>::kElems];
  {
    const __amdgpu_buffer_rsrc_t r0 = k_tile_rsrc<D, BITS>(c, phys, h);
#pragma unroll
    for (int ch = 0; ch < D / Fmt<BITS>::kElems; ++ch)
      kr[ch] = load_stream_buf(r0, static_cast<uint32_t>(lane) * 16u + ch * S * 16);
  }
  static_assert(4 * NQ * VPR <= kThreads, "one query vector per thread");
  if (tid < 4 * NQ * VPR)
    *reinterpret_cast<u32x4_t*>(&qh[qi / VPR / 4][qi / VPR % 4][(qi % VPR) * 8]) = q_ok ? qv : u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  if (w == 0) {  // query norms in fp32
#pragma unroll
    for (int g = 0; g < 4 * NQ; ++g) {
      float s2 = 0.f;
      for (int d = lane; d < D; d += 64) {
        const float x = static_cast<float>(qh[g / 4][g % 4][d]);
        s2 = fmaf(x, x, s2);
      }
      s2 = wave_sum_dpp(s2);
      if (lane == 0) qinv[g] = (g < G && s2 > 0.f) ? 1.f / __builtin_sqrtf(s2) : 0.f;
    }
  }
  __syncthreads();

  const SeqGeom sg = seq_geom(__builtin_amdgcn_readfirstlane(n_seq_lane), c.T, S);
  const int units = min(sg.n_blk, c.max_blocks);
  const size_t cap = static_cast<size_t>(c.max_blocks) * S;
  float* prob = p.prob + static_cast<size_t>(bh) * cap;
  if constexpr (CLAIM) {
    // Claim walk (see the decode's): the first unit is split * 4 + w, then units nsplit * 4 + claim.
    // A unit's chain is claim -> header -> tiles, each given a whole unit of time: at the start of
    // the unit computed in iteration j, the next unit's header and the claim for the one after it
    // (both issued at the start of iteration j - 1) are resolved, that unit's header is requested
    // and the next claim issued; so claims run three units ahead.  The loop has no branch around a
    // memory operation (a claim after one that landed past the end lands past it too, a header
    // past the end is read and ignored), and no store: a store pending beside the loads makes
    // every later wait a wait for all of them (stores and loads share the counter and may complete
    // out of order), so the probabilities of kStage units are staged in LDS and written out
    // together.
    const int base = p.nsplit * kWaves;
    int u = split * kWaves + w;
    if (u >= units) return;  // then units <= base: every claim lands past the end
    int un = base + static_cast<int>(__builtin_amdgcn_readfirstlane(cl));
    int hn = header_load(c, b, un);
    cl = claim_issue(work, lane);
    int nst = 0;
    auto flush = [&]() {
#pragma unroll 1
      for (int k = 0; k < nst; ++k)
        prob[static_cast<size_t>(ustage[w][k]) * S + lane] = pstage[w][k][lane];
      nst = 0;
      // drain here, once per kStage units, so that no store is pending in the loop's other waits
      __builtin_amdgcn_s_waitcnt(0);
    };
    while (u >= 0) {
      const int phys_n = un < units ? header_phys(c, hn) : -1;
      const int un2 = base + static_cast<int>(__builtin_amdgcn_readfirstlane(cl));
      const int hn2 = header_load(c, b, un2);
      cl = claim_issue(work, lane);
      const int nv = min(S, sg.n_cold - u * S);
      const float pr = window_scores<D, G, BITS>(kr, qh, qinv, lane, nv, k_tile_rsrc<D, BITS>(c, phys_n, h));
      // a block without a valid physical id contributes probability 0 (its tokens are never
      // attended); lanes past the last cold token write row entries the selection never reads
      pstage[w][nst][lane] = phys >= 0 && lane < nv ? pr : 0.f;
      if (lane == 0) ustage[w][nst] = u;
      if (++nst == kStage) {
        wave_lds_sync();
        flush();
      }
      u = un < units ? un : -1;
      phys = phys_n;
      un = un2;
      hn = hn2;
    }
    wave_lds_sync();
    flush();
    return;
  }
  int kb = 0;  // walk index of lane 0 of the header batch
  auto phys_of = [&](int k) -> int {
    if (k - kb >= 64) {
      kb = k;
      hb = header_batch(c, b, kb, split, p.nsplit, CU, w, lane);
    }
    return __builtin_amdgcn_readlane(hb, k - kb);
  };
  // the next unit's block id is looked up after this unit's refills are issued, so a header-batch
  // refresh never makes the wave wait for them
  int k = 0;
  int u = walk_unit(0, split, p.nsplit, CU, w);
  int un = walk_unit(1, split, p.nsplit, CU, w);
  int phys_n = u < units && un < units ? phys_of(1) : -1;
  while (u < units) {
    const int nv = min(S, sg.n_cold - u * S);
    const float pr = window_scores<D, G, BITS>(kr, qh, qinv, lane, nv, k_tile_rsrc<D, BITS>(c, phys_n, h));
    // a block without a valid physical id contributes probability 0 (its tokens are never attended)
    if (lane < nv) prob[static_cast<size_t>(u) * S + lane] = phys >= 0 ? pr : 0.f;
    u = un;
    phys = phys_n;
    ++k;
    un = walk_unit(k + 1, split, p.nsplit, CU, w);
    phys_n = un < units ? phys_of(k + 1) : -1;
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
  // every thread sums the wave totals itself (independent LDS reads, no serial pass)
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    const int s = wsum[i];
    before += i < w ? s : 0;
    all += s;
  }
  *total = all;
  __syncthreads();  // wsum is reused by the next scan
  return before + x - v;
}

// Radix select over the key bits [30:0] (keys are fp32 bit patterns of
// probabilities >= 0, so bit 31 is 0 and integer order is value order), in
// three passes of 11, 10 and 10 bits from the top.  Window probabilities share
// their exponent, so a first digit of exponent + 3 mantissa bits still spreads
// them over dozens of bins (8-bit digits put most keys into two or three bins
// and serialise the LDS atomics).
constexpr int kSelPasses = 3;
__device__ __forceinline__ int sel_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int sel_bins(int pass) { return pass == 0 ? 2048 : 1024; }
constexpr int kSelMaxBins = 2048;
// Histogram copies by lane % 16.  Window probabilities crowd into a handful of
// bins, and the lanes of one LDS atomic that hit the same address are applied
// one after another (measured: about 18 us for the first pass over 32768 keys
// with a single copy).  With 16 copies, 4 banks apart, lanes that share a bin
// mostly land on different addresses and banks.  The pick sums the copies.
constexpr int kSelCopies = 16;
constexpr int kSelStride = kSelMaxBins + 4;

__device__ __forceinline__ unsigned* lane_hist(unsigned* hist) {
  return hist + (threadIdx.x & (kSelCopies - 1)) * kSelStride;
}

// Zero the first nb bins (a power of two) of every copy, 16 bytes per store.
__device__ __forceinline__ void clear_hist(unsigned* hist, int nb) {
  const int lg = 29 - __builtin_clz(static_cast<unsigned>(nb));  // log2(nb / 4)
  for (int i = threadIdx.x; i < kSelCopies * (nb >> 2); i += kSelThreads)
    *reinterpret_cast<u32x4_t*>(hist + (i >> lg) * kSelStride + 4 * (i & ((nb >> 2) - 1))) = u32x4_t{0u, 0u, 0u, 0u};
}

// Count of bin i over the copies.
__device__ __forceinline__ unsigned hist_bin(const unsigned* hist, int i) {
  unsigned v = 0;
#pragma unroll
  for (int c = 0; c < kSelCopies; ++c) v += hist[c * kSelStride + i];
  return v;
}

// After a histogram pass: the digit of the krem-th largest key among those
// matching `prefix`, scanning bins from the top digit down (thread t owns the
// bins nb-1-t*bpt ... nb-t*bpt-bpt, in descending order).
__device__ __forceinline__ void radix_pick(const unsigned* hist, int nb, int* wsum, unsigned* s_prefix,
                                           unsigned* s_krem, unsigned prefix, unsigned krem, int shift) {
  const int tid = threadIdx.x;
  const int bpt = nb / kSelThreads;  // 1 or 2
  const int top = nb - 1 - tid * bpt;
  int local = 0;
  unsigned v[2] = {0u, 0u};
  for (int i = 0; i < bpt; ++i) {
    v[i] = hist_bin(hist, top - i);
    local += static_cast<int>(v[i]);
  }
  int total;
  unsigned before = static_cast<unsigned>(block_exclusive_scan(local, wsum, &total));  // keys above my bins
  for (int i = 0; i < bpt; ++i) {
    // the digit whose keys contain the krem-th largest: before < krem <= before + v (unique); the
    // lowest digit takes whatever is left
    if ((before < krem && krem <= before + v[i]) || (top - i == 0 && before < krem && krem > before + v[i])) {
      *s_prefix = prefix | (static_cast<unsigned>(top - i) << shift);
      *s_krem = krem - before;
    }
    before += v[i];
  }
  __syncthreads();
}

// Rows of up to KPT * 1024 keys: every key is loaded into registers once
// (thread t holds keys [t*KPT, t*KPT + KPT), so its indices are contiguous and
// in order), the radix passes run from the registers, and the ordered
// compaction needs two block scans.  Longer rows stream the keys from memory
// on every pass (select_streaming).
constexpr int kSelKPT = 32;

__device__ void select_registers(const unsigned* keys, int n, int K, int32_t* out, unsigned* hist, int* wsum,
                                 unsigned* s_prefix, unsigned* s_krem) {
  constexpr int KPT = kSelKPT;
  const int tid = threadIdx.x;
  const int i0 = tid * KPT;
  // the row is read with coalesced 16-byte loads (vector v * 1024 + t by thread t) and handed over
  // through LDS (rows padded to KPT + 1 words: conflict-free reads) to its owner, thread i / KPT;
  // loading each thread's own 128 contiguous bytes directly makes every load instruction touch 64
  // cache lines and thrashes the L1 (measured: about 6 us for a 32768-key row)
  unsigned* stage = hist;
  {
    const u32x4_t* kv = reinterpret_cast<const u32x4_t*>(keys);  // 16-byte aligned: rows start at multiples of 64 keys
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
      const int vi = v * kSelThreads + tid;  // vector index: keys 4 vi .. 4 vi + 3
      u32x4_t x;
      if (4 * vi + 4 <= n) {
        x = kv[vi];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = 4 * vi + j < n ? keys[4 * vi + j] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * vi + j;
        stage[(i / KPT) * (KPT + 1) + i % KPT] = i < n ? x[j] + 1u : 0u;
      }
    }
  }
  __syncthreads();
  // keys are held as bit pattern + 1 (same order; bit 31 stays 0) and 0 past the row, so every
  // test below against a floor or threshold >= 1 leaves the padding out without a per-key check
  unsigned key[KPT];
#pragma unroll
  for (int k = 0; k < KPT; ++k) key[k] = stage[tid * (KPT + 1) + k];
  __syncthreads();  // the stage is the histogram's memory
  const int nv = max(0, min(KPT, n - i0));  // valid keys of this thread
  // ---- a floor lo <= tau that most keys fall below: if at least K threads hold keys, the
  // first-digit bin of the K-th largest per-thread maximum has K maxima at or above its lower
  // edge, so at least K keys are >= lo and the K-th largest key is too.  Only keys >= lo take
  // part in the radix passes (typically a few percent of the row).
  unsigned lo = 1;
  unsigned tmax = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) tmax = max(tmax, key[k]);
  if (min(kSelThreads, cdiv(n, KPT)) >= K) {  // threads holding keys
    clear_hist(hist, sel_bins(0));
    __syncthreads();
    if (nv > 0) atomicAdd(&lane_hist(hist)[tmax >> sel_shift(0)], 1u);
    __syncthreads();
    radix_pick(hist, sel_bins(0), wsum, s_prefix, s_krem, 0u, static_cast<unsigned>(K), sel_shift(0));
    lo = max(1u, *s_prefix);
    __syncthreads();  // every thread has read the pick before the histogram is cleared again
  }
  // ---- radix select: the K-th largest key (tau) and how many keys equal to it to take
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  for (int pass = 0; pass < kSelPasses; ++pass) {
    const int shift = sel_shift(pass), nb = sel_bins(pass);
    clear_hist(hist, nb);
    __syncthreads();
    unsigned* wh = lane_hist(hist);
#pragma unroll
    for (int k = 0; k < KPT; ++k)
      if (key[k] >= lo && (key[k] & mask) == prefix)
        atomicAdd(&wh[(key[k] >> shift) & static_cast<unsigned>(nb - 1)], 1u);
    __syncthreads();
    radix_pick(hist, nb, wsum, s_prefix, s_krem, prefix, krem, shift);
    prefix = *s_prefix;
    krem = *s_krem;
    mask |= static_cast<unsigned>(nb - 1) << shift;
    __syncthreads();  // every thread has read the pick before the next pass clears the histogram
  }
  const unsigned tau = prefix;
  const int need_eq = static_cast<int>(krem);
  // ---- ordered compaction: every key above tau, and the lowest-index need_eq keys equal to it
  int gt = 0, eq = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    gt += key[k] > tau ? 1 : 0;
    eq += key[k] == tau ? 1 : 0;
  }
  // one scan of both counts (each total is at most 32768, so 16 bits apiece)
  int both_total;
  const int both_before = block_exclusive_scan((gt << 16) | eq, wsum, &both_total);
  const int eq_before = both_before & 0xffff, gt_before = both_before >> 16;
  const int eq_take = max(0, min(eq, need_eq - eq_before));
  int pos = gt_before + min(eq_before, need_eq);  // keys taken by the threads before this one
  int eq_seen = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool is_eq = key[k] == tau;
    const bool take = key[k] > tau || (is_eq && eq_seen < eq_take);
    if (is_eq) ++eq_seen;
    if (take) {
      if (pos < K) out[pos] = i0 + k;
      ++pos;
    }
  }
}

__device__ void select_streaming(const unsigned* keys, int n, int K, int32_t* out, unsigned* hist, int* wsum,
                                 unsigned* s_prefix, unsigned* s_krem) {
  const int tid = threadIdx.x;
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  for (int pass = 0; pass < kSelPasses; ++pass) {
    const int shift = sel_shift(pass), nb = sel_bins(pass);
    clear_hist(hist, nb);
    __syncthreads();
    unsigned* wh = lane_hist(hist);
    for (int i = tid; i < n; i += kSelThreads) {
      const unsigned key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&wh[(key >> shift) & static_cast<unsigned>(nb - 1)], 1u);
    }
    __syncthreads();
    radix_pick(hist, nb, wsum, s_prefix, s_krem, prefix, krem, shift);
    prefix = *s_prefix;
    krem = *s_krem;
    mask |= static_cast<unsigned>(nb - 1) << shift;
    __syncthreads();
  }
  const unsigned tau = prefix;
  const int need_eq = static_cast<int>(krem);
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

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkParams p) {
  constexpr int S = kBlockSize;
  // histogram copies; also the stage of the register path's key hand-over
  constexpr int kLds = kSelCopies * kSelStride > kSelThreads * (kSelKPT + 1) ? kSelCopies * kSelStride
                                                                            : kSelThreads * (kSelKPT + 1);
  __shared__ __attribute__((aligned(16))) unsigned hist[kLds];
  __shared__ int wsum[kSelThreads / 64 + 1];
  __shared__ unsigned s_prefix, s_krem;
  const CacheView& c = p.c;
  const int bh = blockIdx.x;
  const int b = bh / c.H;
  const int tid = threadIdx.x;
  // the score launch before this one is complete: its claim counter goes back to zero
  if (p.work && tid == 0)
    __hip_atomic_store(p.work + static_cast<size_t>(bh) * kClaimStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
  if (n <= kSelKPT * kSelThreads) select_registers(keys, n, K, out, hist, wsum, &s_prefix, &s_krem);
  else select_streaming(keys, n, K, out, hist, wsum, &s_prefix, &s_krem);
}

template <typename Kf>
hipError_t launch_t(Kf kernel, dim3 grid, int block, const TopkParams& p, const LaunchCtx& ctx) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

template <int D, int G, int BITS>
hipError_t launch_tg(const TopkParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  hipError_t e = p.work ? launch_t(topk_score_kernel<D, G, BITS, true>, dim3(p.nsplit, p.c.H, p.c.B), kThreads, p, a)
                        : launch_t(topk_score_kernel<D, G, BITS, false>, dim3(p.nsplit, p.c.H, p.c.B), kThreads, p, a);
  if (e != hipSuccess) return e;
  return launch_t(topk_select_kernel, dim3(p.c.B * p.c.H), kSelThreads, p, b);
}

template <int D, int BITS>
hipError_t launch_tdb(const TopkParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  switch (p.G) {
    case 1: return launch_tg<D, 1, BITS>(p, a, b);
    case 2: return launch_tg<D, 2, BITS>(p, a, b);
    case 4: return launch_tg<D, 4, BITS>(p, a, b);
    case 8: return launch_tg<D, 8, BITS>(p, a, b);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_td(const TopkParams& p, const LaunchCtx& a, const LaunchCtx& b) {
  switch (p.c.bits) {
    case 8: return launch_tdb<D, 8>(p, a, b);
    case 4: return launch_tdb<D, 4>(p, a, b);
    case 0: return launch_tdb<D, 0>(p, a, b);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace detail

using namespace detail;

hipError_t launch_topk(const TopkParams& p, const LaunchCtx& score_ctx, const LaunchCtx& sel_ctx) {
  return p.c.D == 128 ? launch_td<128>(p, score_ctx, sel_ctx) : launch_td<64>(p, score_ctx, sel_ctx);
}

}  // namespace hkv
