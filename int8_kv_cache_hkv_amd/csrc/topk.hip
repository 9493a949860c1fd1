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
        const uint32_t word = word_of(kr[ch], st) ^ kCodeOffsetWord;  // stored offset binary -> signed codes
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

// The kWinTop largest of the wave's 64 keys (unsigned; 0 = no key) and their lanes, wave-uniform,
// in lane order: each of kWinTop rounds takes the wave maximum (DPP inside rows of 16 lanes, then
// the four row results) and retires it in its lowest lane; the retired lanes are then read out in
// ascending order.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_mov_u(unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned x) {
  x = max(x, dpp_mov_u<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp_mov_u<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp_mov_u<0x141>(x));  // row_half_mirror
  x = max(x, dpp_mov_u<0x140>(x));  // row_mirror
  const unsigned a = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 0));
  const unsigned b = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 16));
  const unsigned c = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 32));
  const unsigned d = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(x), 48));
  return max(max(a, b), max(c, d));
}
struct WinTop {
  uint4 k;         // keys of the kWinTop lanes, in lane order
  uint32_t lanes;  // those lanes, 8 bits apiece
};
__device__ __forceinline__ WinTop wave_top(unsigned key, int lane) {
  static_assert(kWinTop == 4, "four keys per window");
  const unsigned orig = key;
  bool taken = false;
#pragma unroll
  for (int r = 0; r < kWinTop; ++r) {
    const unsigned m = wave_max_u32(key);
    const uint64_t hit = __ballot(key == m && !taken);  // never empty: 64 > kWinTop lanes
    if (lane == static_cast<int>(__builtin_ctzll(hit))) {
      key = 0u;
      taken = true;
    }
  }
  uint64_t mask = __ballot(taken);  // exactly kWinTop lanes
  unsigned t[kWinTop], ln = 0u;
#pragma unroll
  for (int r = 0; r < kWinTop; ++r) {
    const int l = static_cast<int>(__builtin_ctzll(mask));
    mask &= mask - 1;
    t[r] = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(orig), l));
    ln |= static_cast<unsigned>(l) << (8 * r);
  }
  return {make_uint4(t[0], t[1], t[2], t[3]), ln};
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
  // claim walk: staged window tops, 20 bytes apiece (kWinTop keys and their lanes), so that four
  // workgroups still fit a CU's LDS
  __shared__ uint4 tstage[CLAIM ? kWaves : 1][CLAIM ? kStage : 1];     // ... their window tops
  __shared__ uint32_t lstage[CLAIM ? kWaves : 1][CLAIM ? kStage : 1];  // ... and those tops' lanes
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
  uint4* wtop = p.wtop + static_cast<size_t>(bh) * c.max_blocks;         // per window: its kWinTop largest keys + 1
  uint32_t* wlane = p.wlane + static_cast<size_t>(bh) * c.max_blocks;    // ... and their lanes
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
      for (int k = 0; k < nst; ++k) {
        prob[static_cast<size_t>(ustage[w][k]) * S + lane] = pstage[w][k][lane];
        if (lane == 0) {
          wtop[ustage[w][k]] = tstage[w][k];
          wlane[ustage[w][k]] = lstage[w][k];
        }
      }
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
      const float pv = phys >= 0 && lane < nv ? pr : 0.f;
      pstage[w][nst][lane] = pv;
      const WinTop tt = wave_top(lane < nv ? __builtin_bit_cast(unsigned, pv) + 1u : 0u, lane);
      if (lane == 0) {
        ustage[w][nst] = u;
        tstage[w][nst] = tt.k;
        lstage[w][nst] = tt.lanes;
      }
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
    const float pv = phys >= 0 ? pr : 0.f;
    if (lane < nv) prob[static_cast<size_t>(u) * S + lane] = pv;
    const WinTop tt = wave_top(lane < nv ? __builtin_bit_cast(unsigned, pv) + 1u : 0u, lane);
    if (lane == 0) {
      wtop[u] = tt.k;
      wlane[u] = tt.lanes;
    }
    u = un;
    phys = phys_n;
    ++k;
    un = walk_unit(k + 1, split, p.nsplit, CU, w);
    phys_n = un < units ? phys_of(k + 1) : -1;
  }
}

// ---------------------------------------------------------------- selection
// The K largest window probabilities of a (sequence, kv-head) row, ties to the lower index, in
// ascending index order.  Keys are the fp32 bit patterns plus one: probabilities are >= 0, so
// integer order is value order, bit 31 stays 0, and 0 is free to mark "no key".
//
// topk_select_kernel: one workgroup per row.  It reads the window tops, not the row:
//  1. a floor lo <= tau (tau: the K-th largest key): at least K keys of the row are >= the K-th
//     largest window top, so the lower edge of the histogram bin holding it is a floor (the bins
//     split the range of the tops into 2048, so lo sits just below tau).
//  2. candidates (every key >= lo) in index order: a window whose smallest top is below lo has all
//     of its keys >= lo among its tops, which are kept in lane order (so in index order); only a
//     window whose tops are all >= lo is read whole (next to none of the 32768-token workload's).
//     Their count is scanned over the workgroup and the candidates are staged in LDS in index order.
//  3. tau and how many keys equal to it to take (radix passes over the range [lo, largest key]):
//     one wave alone when the candidates fit it (no workgroup barrier in the passes), else the
//     whole workgroup; then the ordered output.
// A row of at most kDirectKeys keys is selected from the row itself (then K window tops may not
// exist); a row of more than kTopsWindows windows, or with more than kFinalKeys candidates (keys
// crowded at the floor: many equal keys), by streaming the whole row.
constexpr int kDirectKPT = kDirectKeys / kSelThreads;  // keys per thread of the direct selection
constexpr int kFinalKPT = kFinalKeys / kSelThreads;    // candidates per thread of the block selection
constexpr int kWaveKPT = 16;                            // candidates per lane of the one-wave selection
constexpr int kWaveKeys = 64 * kWaveKPT;
constexpr int kTopsWPT = kTopsWindows / kSelThreads;   // windows per thread
static_assert(kDirectKeys % kSelThreads == 0 && kFinalKeys % kSelThreads == 0 && kTopsWindows % kSelThreads == 0,
              "whole keys per thread");
static_assert(kWinTop * (kDirectKeys / kBlockSize) >= kMaxTopK,
              "a row past kDirectKeys keys has at least K window tops, so the floor exists");
constexpr int kDigitBits = 11;
constexpr int kSelMaxBins = 1 << kDigitBits;
// histogram copies by lane % kSelCopies, 4 banks apart: lanes whose keys share a bin mostly hit
// different addresses (one copy serialises crowded bins); the pick sums the copies
constexpr int kSelCopies = 4;
constexpr int kSelStride = kSelMaxBins + 4;
static_assert(kSelCopies * kSelStride * 4 >= kFinalKeys * 8, "the candidate stage fits the histogram memory");
static_assert(kWaveKeys * 8 + 256 * 4 <= kSelCopies * kSelStride * 4, "one-wave stage and histogram");

struct SelSmem {
  alignas(16) unsigned hist[kSelCopies * kSelStride];  // also the candidate stage
  int wsum[kSelThreads / 64];
  unsigned wred[3][kSelThreads / 64];
  unsigned prefix, krem;
};

// Inclusive prefix sum over the wave's lanes with DPP moves (no LDS): shifts by 1, 2, 4 and 8 inside
// rows of 16 lanes, then lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3.
// Lanes whose source is outside the pattern add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 (rows 1, 3)
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 (rows 2, 3)
  return x;
}

// Exclusive prefix of v over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, SelSmem& sm, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  int before = 0, all = 0;  // every thread sums the wave totals itself (independent LDS reads)
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    const int t = sm.wsum[i];
    before += i < w ? t : 0;
    all += t;
  }
  *total = all;
  __syncthreads();  // wsum is reused by the next scan
  return before + x - v;
}

// Exclusive prefix of v over the wave's lanes; *total gets the sum (wave-uniform).
__device__ __forceinline__ int wave_exclusive_scan(int v, int lane, int* total) {
  const int x = wave_inclusive_scan(v);
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Workgroup minimum and maximum of the nonzero keys and their count (min is ~0u when there is none).
__device__ __forceinline__ void block_min_max_count(unsigned kmin, unsigned kmax, unsigned cnt, SelSmem& sm,
                                                    unsigned* out_min, unsigned* out_max, unsigned* out_cnt) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  kmin = ~wave_max_u32(~kmin);
  kmax = wave_max_u32(kmax);
  cnt = static_cast<unsigned>(wave_sum_dpp(static_cast<float>(cnt)));  // < 2^24: exact in fp32
  if (lane == 0) {
    sm.wred[0][w] = kmin;
    sm.wred[1][w] = kmax;
    sm.wred[2][w] = cnt;
  }
  __syncthreads();
  unsigned a = ~0u, b = 0u, c = 0u;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    a = min(a, sm.wred[0][i]);
    b = max(b, sm.wred[1][i]);
    c += sm.wred[2][i];
  }
  *out_min = a;
  *out_max = b;
  *out_cnt = c;
  __syncthreads();  // wred is reused
}

__device__ __forceinline__ unsigned* lane_hist(SelSmem& sm) {
  return sm.hist + (threadIdx.x & (kSelCopies - 1)) * kSelStride;
}

// Zero the first nb bins (a power of two >= 4) of every copy, 16 bytes per store.
__device__ __forceinline__ void clear_hist(SelSmem& sm, int nb) {
  const int lg = 29 - __builtin_clz(static_cast<unsigned>(nb));  // log2(nb / 4)
  for (int i = threadIdx.x; i < kSelCopies * (nb >> 2); i += kSelThreads)
    *reinterpret_cast<u32x4_t*>(sm.hist + (i >> lg) * kSelStride + 4 * (i & ((nb >> 2) - 1))) =
        u32x4_t{0u, 0u, 0u, 0u};
}

// After a histogram pass over the kSelMaxBins bins: the digit of the krem-th largest counted key,
// scanning bins from the top digit down (thread t owns bins 4 (511 - t) .. 4 (511 - t) + 3, read
// as one 16-byte vector per copy).  Sets sm.prefix = prefix | digit << shift and sm.krem = its rank
// among the keys of that digit.  A krem beyond the counted keys takes digit 0.
constexpr int kPickBins = kSelMaxBins / kSelThreads;
static_assert(kPickBins == 4, "one 16-byte vector of bins per thread and copy");
__device__ __forceinline__ void radix_pick(SelSmem& sm, unsigned prefix, unsigned krem, int shift) {
  const int tid = threadIdx.x;
  const int b0 = kSelMaxBins - kPickBins * (tid + 1);  // lowest bin of this thread
  u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < kSelCopies; ++c) v += *reinterpret_cast<const u32x4_t*>(&sm.hist[c * kSelStride + b0]);
  const int local = static_cast<int>(v[0] + v[1] + v[2] + v[3]);
  int total;
  unsigned before = static_cast<unsigned>(block_exclusive_scan(local, sm, &total));  // keys above my bins
#pragma unroll
  for (int i = kPickBins - 1; i >= 0; --i) {
    const int bin = b0 + i;
    if ((before < krem && krem <= before + v[i]) || (bin == 0 && before < krem && krem > before + v[i])) {
      sm.prefix = prefix | (static_cast<unsigned>(bin) << shift);
      sm.krem = krem - before;
    }
    before += v[i];
  }
  __syncthreads();
}

// Radix select over keys held in registers across the workgroup (0 = none): the K-th largest key
// among those >= base, by digits of (key - base) below bit `bits` (every counted key - base is
// < 2^bits), 11 bits per pass from the top, at most max_passes passes.  Returns base + the selected
// digits (the lower edge of the last bin) and, in *krem, the rank of the K-th largest among the keys
// of that bin.  With every pass run, that is tau itself and *krem the number of keys equal to tau
// among the K largest.
template <int KPT>
__device__ unsigned range_select(const unsigned (&key)[KPT], unsigned base, int bits, int K, int max_passes,
                                 SelSmem& sm, int* krem_out) {
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  int hi = bits;
  for (int pass = 0; pass < max_passes && hi > 0; ++pass) {
    const int wd = min(kDigitBits, hi);
    const int shift = hi - wd;
    const unsigned dm = (1u << wd) - 1u;  // digit mask (bins past it stay empty)
    clear_hist(sm, kSelMaxBins);
    __syncthreads();
    unsigned* wh = lane_hist(sm);
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const unsigned r = key[k] - base;
      if (key[k] >= base && key[k] != 0u && (r & mask) == prefix) atomicAdd(&wh[(r >> shift) & dm], 1u);
    }
    __syncthreads();
    radix_pick(sm, prefix, krem, shift);
    prefix = sm.prefix;
    krem = sm.krem;
    mask |= dm << shift;
    hi = shift;
    __syncthreads();  // every thread has read the pick before the next pass clears the histogram
  }
  *krem_out = static_cast<int>(krem);
  return base + prefix;
}

// The same selection by one wave over the keys its lanes hold, in 8-bit digits (256 bins, four
// per lane: a pass is a few dozen instructions), with a histogram of its own in LDS (hist: 256 words
// no other wave touches).  Every pass stays inside the wave.
constexpr int kWaveDigitBits = 8;
constexpr int kWaveBins = 1 << kWaveDigitBits;
template <int KPT>
__device__ unsigned wave_range_select(const unsigned (&key)[KPT], unsigned base, int bits, int K, unsigned* hist,
                                      int lane, int* krem_out) {
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  int hi = bits;
  constexpr int BPL = kWaveBins / 64;  // lane l owns bins 4 (63 - l) .. 4 (63 - l) + 3
  static_assert(BPL == 4, "one 16-byte vector of bins per lane");
  const int b0 = kWaveBins - BPL * (lane + 1);
  while (hi > 0) {
    const int wd = min(kWaveDigitBits, hi);
    const int shift = hi - wd;
    const unsigned dm = (1u << wd) - 1u;  // digit mask (bins past it stay empty)
    *reinterpret_cast<u32x4_t*>(&hist[b0]) = u32x4_t{0u, 0u, 0u, 0u};
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      const unsigned r = key[k] - base;
      if (key[k] >= base && key[k] != 0u && (r & mask) == prefix) atomicAdd(&hist[(r >> shift) & dm], 1u);
    }
    wave_lds_sync();
    const u32x4_t hv = *reinterpret_cast<const u32x4_t*>(&hist[b0]);
    const int local = static_cast<int>(hv[0] + hv[1] + hv[2] + hv[3]);
    int total;
    const unsigned before = static_cast<unsigned>(wave_exclusive_scan(local, lane, &total));
    // the lane whose bins hold the krem-th largest (or, past the counted keys, lane 63: bin 0)
    const bool mine = (before < krem && krem <= before + static_cast<unsigned>(local)) ||
                      (lane == 63 && krem > before + static_cast<unsigned>(local));
    const uint64_t who = __ballot(mine);
    const int at = static_cast<int>(__builtin_ctzll(who));  // never empty
    unsigned digit = 0, kr = krem, bf = before;
    bool found = false;
#pragma unroll
    for (int i = BPL - 1; i >= 0; --i) {
      const bool hit = !found && ((bf < krem && krem <= bf + hv[i]) || b0 + i == 0);
      digit = hit ? static_cast<unsigned>(b0 + i) : digit;
      kr = hit ? krem - bf : kr;
      found = found || hit;
      bf += hv[i];
    }
    digit = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(digit), at));
    krem = static_cast<unsigned>(__builtin_amdgcn_readlane(static_cast<int>(kr), at));
    prefix |= digit << shift;
    mask |= dm << shift;
    hi = shift;
    wave_lds_sync();  // the next pass clears the bins this one read
  }
  *krem_out = static_cast<int>(krem);
  return base + prefix;
}

// Bits of the range of keys in [lo, hi]: every key - lo < 2^result.
__device__ __forceinline__ int range_bits(unsigned lo, unsigned hi) {
  return hi > lo ? 32 - __builtin_clz(hi - lo) : 0;
}

// (greater << 16 | equal) counts of one holder's keys against tau (each total is below 65536).
template <int KPT>
__device__ __forceinline__ int count_both(const unsigned (&key)[KPT], unsigned tau, int* eq_out) {
  int gt = 0, eq = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    gt += key[k] > tau ? 1 : 0;
    eq += key[k] == tau ? 1 : 0;
  }
  *eq_out = eq;
  return (gt << 16) | eq;
}

// Output positions of one holder's keys (held in list order): every key above tau and the first
// need_eq keys equal to it are taken; both_before is the (greater << 16 | equal) count of the
// holders before this one.  Writes out[pos] = idx for each taken key with pos < K.
template <int KPT>
__device__ __forceinline__ void take_keys(const unsigned (&key)[KPT], const int (&idx)[KPT], unsigned tau,
                                          int need_eq, int K, int both_before, int eq, int32_t* out) {
  const int eq_before = both_before & 0xffff, gt_before = both_before >> 16;
  const int eq_take = max(0, min(eq, need_eq - eq_before));
  int pos = gt_before + min(eq_before, need_eq);  // keys taken by the holders before this one
  int eq_seen = 0;
#pragma unroll
  for (int k = 0; k < KPT; ++k) {
    const bool is_eq = key[k] == tau;
    const bool take = key[k] > tau || (is_eq && eq_seen < eq_take);
    if (is_eq) ++eq_seen;
    if (take) {
      if (pos < K) out[pos] = idx[k];
      ++pos;
    }
  }
}

// The whole row streamed from memory on every pass (three fixed 11/10/10-bit digits of the key).
__device__ void select_streaming(const unsigned* prob_bits, int n, int K, int32_t* out, SelSmem& sm) {
  const int tid = threadIdx.x;
  unsigned prefix = 0, mask = 0, krem = static_cast<unsigned>(K);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
    const unsigned dm = pass == 0 ? 2047u : 1023u;
    clear_hist(sm, kSelMaxBins);
    __syncthreads();
    unsigned* wh = lane_hist(sm);
    for (int i = tid; i < n; i += kSelThreads) {
      const unsigned key = prob_bits[i] + 1u;
      if ((key & mask) == prefix) atomicAdd(&wh[(key >> shift) & dm], 1u);
    }
    __syncthreads();
    radix_pick(sm, prefix, krem, shift);
    prefix = sm.prefix;
    krem = sm.krem;
    mask |= dm << shift;
    __syncthreads();
  }
  const unsigned tau = prefix;
  const int need_eq = static_cast<int>(krem);
  int carry_sel = 0, carry_eq = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + tid;
    const unsigned key = i < n ? prob_bits[i] + 1u : 0u;
    const int is_eq = key == tau ? 1 : 0;
    const int is_gt = key > tau ? 1 : 0;
    int eq_total;
    const int eq_excl = block_exclusive_scan(is_eq, sm, &eq_total);
    const int take = (is_gt || (is_eq && carry_eq + eq_excl < need_eq)) ? 1 : 0;
    int sel_total;
    const int sel_excl = block_exclusive_scan(take, sm, &sel_total);
    if (take && carry_sel + sel_excl < K) out[carry_sel + sel_excl] = i;
    carry_eq += eq_total;
    carry_sel += sel_total;
  }
}

// Key `lane` of window wi of a row (0 past the row's n): a whole window is read by one wave, one
// coalesced 4-byte load per lane (lane = token of the window).
static_assert(kBlockSize == 64, "a window is one key per lane");
__device__ __forceinline__ unsigned window_key(const unsigned* pb, int wi, int n, int lane) {
  const int i = wi * kBlockSize + lane;
  return i < n ? pb[i] + 1u : 0u;
}

// Whole windows a wave keeps in registers between the count and the stage (one key per lane and
// window); any further whole window of the wave is read again for the stage.
constexpr int kHeldWhole = 4;

__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(TopkParams p) {
  constexpr int S = kBlockSize;
  __shared__ SelSmem sm;
  const CacheView& c = p.c;
  const int bh = blockIdx.x;
  const int b = bh / c.H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // the score launch before this one is complete: its claim counter goes back to zero
  if (p.work && tid == 0)
    __hip_atomic_store(p.work + static_cast<size_t>(bh) * kClaimStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const SeqGeom sg = seq_geom(c.seq_len[b], c.T, S);
  const int n = min(sg.n_cold, c.max_blocks * S);  // never read past this (sequence, head)'s row
  const int K = p.k;
  int32_t* out = p.out_idx + static_cast<size_t>(bh) * K;
  const size_t cap = static_cast<size_t>(c.max_blocks) * S;
  const unsigned* pb = reinterpret_cast<const unsigned*>(p.prob + static_cast<size_t>(bh) * cap);

  if (n <= K) {
    for (int i = tid; i < K; i += kSelThreads) out[i] = i < n ? i : -1;
    return;
  }
  const int nw = cdiv(n, S);
  if (n <= kDirectKeys) {  // from the row (thread t: keys [t KPT, t KPT + KPT))
    unsigned key[kDirectKPT];
    int idx[kDirectKPT];
#pragma unroll
    for (int k = 0; k < kDirectKPT; ++k) {
      const int i = tid * kDirectKPT + k;
      key[k] = i < n ? pb[i] + 1u : 0u;
      idx[k] = i;
    }
    int need_eq;
    const unsigned tau = range_select<kDirectKPT>(key, 1u, 31, K, 3, sm, &need_eq);
    int eq, tot;
    const int both = count_both<kDirectKPT>(key, tau, &eq);
    const int before = block_exclusive_scan(both, sm, &tot);
    take_keys<kDirectKPT>(key, idx, tau, need_eq, K, before, eq, out);
    return;
  }
  if (nw > kTopsWindows) {
    select_streaming(pb, n, K, out, sm);
    return;
  }
  // ---- 1. the floor.  Thread t holds windows t + 512 v (v < kTopsWPT), so every thread has work in
  // the first round and the later rounds are skipped as a whole when the row is short.
  const uint4* tops = p.wtop + static_cast<size_t>(bh) * c.max_blocks;
  const uint32_t* lanes = p.wlane + static_cast<size_t>(bh) * c.max_blocks;
  constexpr int WT = kWinTop;
  const int rounds = cdiv(nw, kSelThreads);  // (workgroup-uniform)
  unsigned tk[WT * kTopsWPT];
  uint32_t tl[kTopsWPT];
  static_assert(WT == 4, "a window's tops are one 16-byte vector");
#pragma unroll
  for (int v = 0; v < kTopsWPT; ++v) {
    const int wi = v * kSelThreads + tid;
    const bool ok = v < rounds && wi < nw;
    const uint4 a = ok ? tops[wi] : make_uint4(0u, 0u, 0u, 0u);
    tl[v] = ok ? lanes[wi] : 0u;
    tk[WT * v + 0] = a.x;
    tk[WT * v + 1] = a.y;
    tk[WT * v + 2] = a.z;
    tk[WT * v + 3] = a.w;
  }
  unsigned tmin = ~0u, tmax = 0u, tcnt = 0u;
#pragma unroll
  for (int k = 0; k < WT * kTopsWPT; ++k) {
    if (tk[k] != 0u) {
      tmin = min(tmin, tk[k]);
      tmax = max(tmax, tk[k]);
      ++tcnt;
    }
  }
  unsigned bmin, kmax, bcnt;
  block_min_max_count(tmin, tmax, tcnt, sm, &bmin, &kmax, &bcnt);
  int unused;
  // (bcnt >= K: a row of more than kDirectKeys keys has more than kWinTop kDirectKeys / 64 >= K tops)
  const int fbits = range_bits(bmin, kmax);
  const unsigned lo = max(1u, range_select<WT * kTopsWPT>(tk, bmin, fbits, K, 1, sm, &unused));
  // the floor's bin [lo, band_hi): fewer than K tops lie above it, so tau lies in it unless the keys
  // of whole windows push it higher
  const int fshift = max(0, fbits - kDigitBits);
  const unsigned band_hi = lo + (1u << fshift);
  // ---- 2. the candidates of each round's windows (one window per thread), counted, scanned and
  // staged in index order
  uint64_t* stage = reinterpret_cast<uint64_t*>(sm.hist);
  int m_all = 0;
  for (int v = 0; v < rounds; ++v) {
    const int wi = v * kSelThreads + tid;
    unsigned kv[WT];
    unsigned tmn = ~0u;
#pragma unroll
    for (int r = 0; r < WT; ++r) {
      kv[r] = 0u;
#pragma unroll
      for (int u = 0; u < kTopsWPT; ++u) kv[r] = u == v ? tk[WT * u + r] : kv[r];
      tmn = min(tmn, kv[r]);
    }
    uint32_t lv = tl[0];
#pragma unroll
    for (int u = 1; u < kTopsWPT; ++u) lv = u == v ? tl[u] : lv;
    const bool whole = wi < nw && tmn >= lo;  // every top >= lo: more keys may be
    int nc = 0;
#pragma unroll
    for (int r = 0; r < WT; ++r) nc += !whole && kv[r] >= lo ? 1 : 0;
    // whole windows (next to none; the short last window of a row is one): the wave reads each of
    // its threads' whole windows together, lane j holding key j, and counts it with a ballot
    const uint64_t wmask = __ballot(whole);  // (wave-uniform)
    const int wbase = v * kSelThreads + w * 64;  // window of lane 0's thread
    unsigned held[kHeldWhole];
#pragma unroll
    for (int k = 0; k < kHeldWhole; ++k) held[k] = 0u;
    {
      uint64_t m = wmask;
      for (int k = 0; m != 0ull; ++k) {
        const int owner = __builtin_ctzll(m);
        m &= m - 1ull;
        const unsigned key = window_key(pb, wbase + owner, n, lane);
        const int cnt = __builtin_popcountll(__ballot(key >= lo));
        nc += lane == owner ? cnt : 0;
#pragma unroll
        for (int j = 0; j < kHeldWhole; ++j) held[j] = j == k ? key : held[j];
      }
    }
    int tot;
    int pos = m_all + block_exclusive_scan(nc, sm, &tot);
    if (m_all + tot > kFinalKeys) {  // (uniform)
      select_streaming(pb, n, K, out, sm);
      return;
    }
    if (!whole) {
#pragma unroll
      for (int r = 0; r < WT; ++r) {
        const unsigned ln = (lv >> (8 * r)) & 63u;
        if (kv[r] >= lo)  // (a window past the row has no keys: its tops are 0)
          stage[pos++] = static_cast<uint64_t>(kv[r]) |
                         (static_cast<uint64_t>(static_cast<uint32_t>(wi * S + static_cast<int>(ln))) << 32);
      }
    }
    {
      // a whole window's kept keys in index order: from its owner's position, each lane at the
      // rank of its key among the window's kept keys
      uint64_t m = wmask;
      for (int k = 0; m != 0ull; ++k) {
        const int owner = __builtin_ctzll(m);
        m &= m - 1ull;
        unsigned key = 0u;
#pragma unroll
        for (int j = 0; j < kHeldWhole; ++j) key = j == k ? held[j] : key;
        if (k >= kHeldWhole) key = window_key(pb, wbase + owner, n, lane);
        const bool keep = key >= lo;
        const uint64_t km = __ballot(keep);
        const int at = __builtin_amdgcn_readlane(pos, owner) +
                       static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(km >> 32),
                                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(km), 0u)));
        if (keep)
          stage[at] = static_cast<uint64_t>(key) |
                      (static_cast<uint64_t>(static_cast<uint32_t>((wbase + owner) * S + lane)) << 32);
      }
    }
    m_all += tot;
  }
  __syncthreads();
  // ---- 3. tau among the candidates, then the ordered output
  if (m_all <= kWaveKeys) {  // one wave (lane l: candidates [l KPT, l KPT + KPT))
    if (w != 0) return;
    unsigned key[kWaveKPT];
    int idx[kWaveKPT];
#pragma unroll
    for (int k = 0; k < kWaveKPT; ++k) {
      const int j = lane * kWaveKPT + k;
      const uint64_t e = j < m_all ? stage[j] : 0ull;
      key[k] = static_cast<unsigned>(e);
      idx[k] = static_cast<int>(e >> 32);
    }
    unsigned* whist = sm.hist + 2 * kWaveKeys;  // past the stage (words)
    int above = 0;
#pragma unroll
    for (int k = 0; k < kWaveKPT; ++k) above += key[k] >= band_hi ? 1 : 0;
    int n_above;
    (void)wave_exclusive_scan(above, lane, &n_above);
    int need_eq;
    unsigned tau;
    if (n_above < K) {  // tau is in the floor's bin: select among the keys inside it only
      unsigned kb[kWaveKPT];
#pragma unroll
      for (int k = 0; k < kWaveKPT; ++k) kb[k] = key[k] < band_hi ? key[k] : 0u;
      tau = wave_range_select<kWaveKPT>(kb, lo, fshift, K - n_above, whist, lane, &need_eq);
    } else {
      tau = wave_range_select<kWaveKPT>(key, lo, range_bits(lo, kmax), K, whist, lane, &need_eq);
    }
    int eq, tot;
    const int both = count_both<kWaveKPT>(key, tau, &eq);
    const int before = wave_exclusive_scan(both, lane, &tot);
    take_keys<kWaveKPT>(key, idx, tau, need_eq, K, before, eq, out);
    return;
  }
  unsigned key[kFinalKPT];
  int idx[kFinalKPT];
#pragma unroll
  for (int k = 0; k < kFinalKPT; ++k) {
    const int j = tid * kFinalKPT + k;
    const uint64_t e = j < m_all ? stage[j] : 0ull;
    key[k] = static_cast<unsigned>(e);
    idx[k] = static_cast<int>(e >> 32);
  }
  int above = 0;
#pragma unroll
  for (int k = 0; k < kFinalKPT; ++k) above += key[k] >= band_hi ? 1 : 0;
  int n_above;
  (void)block_exclusive_scan(above, sm, &n_above);  // (its barriers also end the reads of the stage,
                                                    // which is the histogram's memory)
  int need_eq;
  unsigned tau;
  if (n_above < K) {  // tau is in the floor's bin: select among the keys inside it only
    unsigned kb[kFinalKPT];
#pragma unroll
    for (int k = 0; k < kFinalKPT; ++k) kb[k] = key[k] < band_hi ? key[k] : 0u;
    tau = range_select<kFinalKPT>(kb, lo, fshift, K - n_above, 3, sm, &need_eq);
  } else {
    tau = range_select<kFinalKPT>(key, lo, range_bits(lo, kmax), K, 3, sm, &need_eq);
  }
  int eq, tot;
  const int both = count_both<kFinalKPT>(key, tau, &eq);
  const int before = block_exclusive_scan(both, sm, &tot);
  take_keys<kFinalKPT>(key, idx, tau, need_eq, K, before, eq, out);
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
