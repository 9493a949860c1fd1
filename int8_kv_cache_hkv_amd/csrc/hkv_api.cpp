// Host side of the libhkv C ABI: protocol validation, size queries, launch
// planning (from the host seq_len mirror) and kernel timing.
//
// Protocol rules (Hybrid KV Cache page, 3.1 and 5.1): hot_tokens is a power of
// two in {16, 32, 64, 128}; block_size is a positive multiple of 8;
// quantization_bits is 4 or 8 (5.2 adds 0 = FP16 cold zone); all three widths
// are built (block_size 64 and head_dim 64 / 128 only).  The pages
// describe a launch-time CUDA_ERROR_INVALID_VALUE for violations; here every
// check runs on the host before any HIP call.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "hkv.h"
#include "hkv_internal.h"

namespace hkv {

template <int D, int BITS>
hipError_t launch_decode_db(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order) {
  switch (p.G) {
    case 1: return launch_decode_dgb<D, 1, BITS>(p, ctx, order);
    case 2: return launch_decode_dgb<D, 2, BITS>(p, ctx, order);
    case 4: return launch_decode_dgb<D, 4, BITS>(p, ctx, order);
    case 8: return launch_decode_dgb<D, 8, BITS>(p, ctx, order);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_decode_b(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order) {
  return p.c.D == 128 ? launch_decode_db<128, BITS>(p, ctx, order) : launch_decode_db<64, BITS>(p, ctx, order);
}

hipError_t launch_decode(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order) {
  switch (p.c.bits) {
    case 8: return launch_decode_b<8>(p, ctx, order);
    case 4: return launch_decode_b<4>(p, ctx, order);
    case 0: return launch_decode_b<0>(p, ctx, order);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hkv

struct hkv_ctx {
  int H, D, T, S, bits;
  int force_splits = 0;      // plan override (hkv_plan_override): static plans of this many splits
  int claim_workgroups = 0;  // plan override: grid of claim plans (0 = the width's default)
  bool timing = false;
  unsigned long long* stamps = nullptr;  // phase timestamps (hkv_phase_stamps), nullptr = off
  size_t stamp_wgs = 0;
  struct Pending {
    int kind;
    hipEvent_t start, stop;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> free_events;
  double total_ms[HKV_KERNEL_KINDS] = {};
  int64_t count[HKV_KERNEL_KINDS] = {};
};

namespace {

using hkv::LaunchCtx;

// Target workgroups per decode/top-K launch: 4 per CU on 256 CUs, 16 waves/CU.
constexpr int kTargetWorkgroups = 1024;
// Claim plans (see plan_splits) target 2 workgroups per CU: with fewer waves in flight the loaded
// memory latency is shorter, and so is the tail of units the waves have claimed ahead (131072-token
// step, measured: 1024 -> 178, 768 -> 174, 512 -> 171, 384 -> 175, 256 -> 224 us).
constexpr int kClaimTargetWorkgroups = 512;
constexpr int kTopkClaimTargetWorkgroups = 1024;
// Small launches (at most kSmallLaunchUnits cold units in all) are latency-bound: fewer workgroups,
// each wave walking several units with the next one's tiles in flight, and static splits
// (2048-token fused step, measured over batch 4 / 8 / 16: 14.4 / 16.4 / 22.3 us with the 1024
// target; 14.0 / 15.5 us with 256, batch 16 above the threshold).
constexpr int64_t kSmallLaunchUnits = 2048;
constexpr int kSmallTargetWorkgroups = 256;
using hkv::kMaxSplits;

bool valid_protocol(int hot_tokens, int block_size) {
  const bool hot_ok = hot_tokens == 16 || hot_tokens == 32 || hot_tokens == 64 || hot_tokens == 128;
  return hot_ok && block_size > 0 && block_size % 8 == 0;
}

int64_t cold_blocks(int64_t tokens, int T, int S) {
  const int64_t n_cold = std::max<int64_t>(0, tokens - T);
  return (n_cold + S - 1) / S;
}

// Split plan: units per split is a multiple of the 4 waves of a workgroup and
// a split count never exceeds kMaxSplits.
//  * When the launch fits the resident workgroup slots (about kTargetWorkgroups),
//    all of its workgroups (cold splits + the extra_parts other workgroups of
//    each (sequence, kv-head): hot zone, and the tail block of a fused append)
//    are sized to be resident at once: a straggler that starts late delays the
//    merge of its (sequence, kv-head).
//  * With more (sequence, kv-head) pairs than that (large ragged batches), the
//    grid cannot be resident anyway: short splits of kBatchSplitUnits units are
//    scheduled as slots free up, so a long sequence does not leave one
//    workgroup streaming alone at the end.
constexpr int64_t kBatchSplitUnits = 32;
struct SplitPlan {
  int nsplit;
  int per_split;
  int wg_order;   // workgroup order of the grid (see wg_coord)
  int claim;      // resident plans with long splits claim their units dynamically (dense decode)
  int batch;      // batch plan: splits of kBatchSplitUnits, scheduled as resident slots free up
};
SplitPlan plan_splits(int64_t bh, int64_t units, int extra_parts = 1, int64_t target_wg = kTargetWorkgroups,
                      int64_t claim_target_wg = kClaimTargetWorkgroups) {
  units = std::max<int64_t>(1, units);
  const int64_t target = target_wg / bh - extra_parts;
  int64_t per = target >= 2 ? hkv::kWaves * ((units + hkv::kWaves * target - 1) / (hkv::kWaves * target))
                            : kBatchSplitUnits;
  int64_t ns = (units + per - 1) / per;
  if (ns > kMaxSplits) {
    per = hkv::kWaves * ((units + hkv::kWaves * kMaxSplits - 1) / (hkv::kWaves * kMaxSplits));
    ns = (units + per - 1) / per;
  }
  // plans with long splits claim their units dynamically (static splits of equal size were measured
  // to finish up to 6x apart); resident ones on a grid of kClaimTargetWorkgroups in split-major
  // order.  Batch plans claim too: a sequence's splits that start in different rounds of the
  // resident slots then share its blocks (ragged fused step, measured: 124.6 -> 122.0 us)
  const int claim = claim_target_wg > 0 && per >= hkv::kClaimUnits ? 1 : 0;
  if (claim && target >= 2) {
    const int64_t tc = std::max<int64_t>(2, claim_target_wg / bh - extra_parts);
    if (tc < ns) {  // only ever fewer splits (ns <= kMaxSplits holds)
      per = hkv::kWaves * ((units + hkv::kWaves * tc - 1) / (hkv::kWaves * tc));
      ns = (units + per - 1) / per;
    }
  }
  const int order = (claim && target >= 2) ? hkv::kOrderSplitMajor : hkv::kOrderPlain;
  return {static_cast<int>(ns), static_cast<int>(per), order, claim, target < 2 ? 1 : 0};
}

// Workgroups of a claim plan's grid (2 per CU at 8 bits: fewer waves in flight keep the loaded
// latency and the tail of claimed-ahead units short).  A 4-bit unit is half an 8-bit one: its
// grid is doubled so that as many bytes stay in flight.
int64_t claim_target(const hkv_ctx* h) {
  if (h->claim_workgroups > 0) return h->claim_workgroups;
  return h->bits == 4 ? 2 * kClaimTargetWorkgroups : kClaimTargetWorkgroups;
}

int64_t units_sum(const std::vector<int64_t>& units) {
  int64_t t = 0;
  for (int64_t u : units) t += u;
  return t;
}

// Plan of a dense decode or fused step over bh (sequence, kv-head) pairs of at most units_max units.
SplitPlan dense_plan(const hkv_ctx* h, int64_t bh, int64_t units_max, int64_t units_total, int extra_parts) {
  if (units_total <= kSmallLaunchUnits)
    return plan_splits(bh, units_max, extra_parts, kSmallTargetWorkgroups, 0);
  return plan_splits(bh, units_max, extra_parts, kTargetWorkgroups, claim_target(h));
}

// Static plan of n splits (plan override): units per split a multiple of the 4 waves, plain order.
SplitPlan forced_plan(int64_t units, int n) {
  units = std::max<int64_t>(1, units);
  const int64_t per = hkv::kWaves * ((units + hkv::kWaves * n - 1) / (hkv::kWaves * n));
  return {static_cast<int>((units + per - 1) / per), static_cast<int>(per), hkv::kOrderPlain, 0, 0};
}

// The decode variant that carries the entropy statistic runs static plans in plain order only:
// with the statistic asked for, a claim or batch plan becomes the static plan of as many splits.
SplitPlan stats_plan(const hkv_cache_desc* c, const SplitPlan& sp, int64_t units) {
  if (!c->entropy || (!sp.claim && !sp.batch && sp.wg_order == hkv::kOrderPlain)) return sp;
  return forced_plan(units, sp.nsplit);
}

// Upper bound of the split count of plan_splits over every unit count in
// [1, units_cap] and extra_parts >= 1: a resident plan has at most
// kTargetWorkgroups / bh - 1 splits and at most ceil(units / 4); a batch plan
// ceil(units / kBatchSplitUnits); both capped by kMaxSplits.
int max_splits(int64_t bh, int64_t units_cap) {
  const int64_t u = std::max<int64_t>(1, units_cap);
  const int64_t resident = std::min<int64_t>(std::max<int64_t>(1, kTargetWorkgroups / bh - 1), (u + 3) / 4);
  const int64_t batch = (u + kBatchSplitUnits - 1) / kBatchSplitUnits;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kMaxSplits, std::max(resident, batch))));
}

// Sparse decode: one unit of kSparseUnit selected tokens per wave, so every
// gather chain of a call runs concurrently (k_sel <= kMaxTopK keeps this to a
// few splits per (sequence, kv-head)).
// Batch plans run in several rounds of the resident slots; a split that starts in the last round
// with a full run of blocks ends long after the rest (a list-scheduling model of the 64-sequence
// ragged batch: makespan 1.6x the mean slot load in sequence order, 1.2x longest first).  So the
// table lists the cold-split groups by their block count, most first (ties: sequence, split), and
// puts the short hot-zone (and append) groups, which every merge needs, after the cold groups that
// fill the resident slots once: placed first, their latency-bound workgroups held every slot at
// the start (ragged fused step, measured: short groups first 133 us, after 64 / 96 / 128 / 160 /
// 192 cold groups 128 / 128 / 124 / 124 / 127 us, last 130 us; sequence order 141 us).
// After the resident slots' first fill, the hot-zone groups are ordered among the remaining cold
// groups as if each were kHotGroupUnits blocks long (a fused step's append workgroup takes 14-17 us
// under load; ragged fused step, measured: weight 4 / 8 / 12 / 16 / 20 -> 107.9 / 106.7 / 106.2 /
// 106.5 / 107.1 us, all after the cold groups 107.0 us).
// units[b]: the blocks of sequence b this launch attends.  Returns false (plain order kept) when
// the table cannot hold the groups.
// Only the cold splits a sequence takes part with are listed (hkv::table_splits of its unit count;
// the kernel derives the same count), so a sequence's merge never waits for a split that would only
// have found its units taken.  Sets p.order_groups.
constexpr int64_t kHotGroupUnits = 12;
bool order_by_work(hkv::DecodeParams& p, const std::vector<int64_t>& units, int64_t per, uint16_t* order) {
  const int B = static_cast<int>(units.size());
  // entries are (sequence << 7 | part) in 16 bits
  const int parts = hkv::grid_parts(p);
  if (static_cast<int64_t>(B) * parts > hkv::kOrderTableMax || B > 511 || parts > 128) return false;
  std::vector<std::pair<int64_t, int>> v;
  v.reserve(static_cast<size_t>(B) * p.nsplit);
  for (int b = 0; b < B; ++b)
    for (int s = 0; s < hkv::table_splits(p.nsplit, static_cast<int>(per), units[b]); ++s)
      v.push_back({-std::max<int64_t>(0, std::min<int64_t>(per, units[b] - s * per)), (b << 7) | s});
  std::stable_sort(v.begin(), v.end(), [](const auto& x, const auto& y) { return x.first < y.first; });
  const size_t at = std::min<size_t>(kTargetWorkgroups / p.c.H, v.size());
  size_t i = 0;
  for (size_t k = 0; k < at; ++k) order[i++] = static_cast<uint16_t>(v[k].second);
  // the hot-zone (and append) groups join the remaining cold groups in the same longest-first order,
  // weighted as kHotGroupUnits blocks each
  std::vector<std::pair<int64_t, int>> rest(v.begin() + at, v.end());
  for (int b = 0; b < B; ++b)
    for (int s = p.nsplit; s < parts; ++s) rest.push_back({-kHotGroupUnits, (b << 7) | s});
  std::stable_sort(rest.begin(), rest.end(), [](const auto& x, const auto& y) { return x.first < y.first; });
  for (const auto& e : rest) order[i++] = static_cast<uint16_t>(e.second);
  p.order_groups = static_cast<int>(i);
  return true;
}

SplitPlan plan_sparse(int k_sel) {
  const int units = std::max(1, (k_sel + hkv::kSparseUnit - 1) / hkv::kSparseUnit);
  return {(units + hkv::kWaves - 1) / hkv::kWaves, hkv::kWaves, 0};
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of one (block, kv-head, K|V) cold tile: S x D codes of 8 or 4 bits, or fp16 values.
size_t tile_bytes(const hkv_ctx* h) {
  const size_t elems = static_cast<size_t>(h->S) * h->D;
  return h->bits == 0 ? elems * 2 : elems * h->bits / 8;
}

// Compacted sparse store: counts int32 [B*H], then (256-byte aligned) the per-token scales float2
// [B*H][U][64], then (256-byte aligned) the units [B*H][U][2][tile bytes]; U = ceil(k_sel / 64).
struct StoreLayout {
  int units;
  size_t scales_off, units_off, bytes;
};
StoreLayout store_layout(const hkv_ctx* h, int batch, int k_sel) {
  StoreLayout l;
  l.units = (k_sel + hkv::kBlockSize - 1) / hkv::kBlockSize;
  const size_t bh = static_cast<size_t>(batch) * h->H;
  l.scales_off = align_up(bh * sizeof(int32_t), 256);
  l.units_off = align_up(l.scales_off + bh * l.units * hkv::kBlockSize * 2 * sizeof(float), 256);
  l.bytes = l.units_off + bh * l.units * 2 * tile_bytes(h);
  return l;
}

hkv_status check_desc(const hkv_ctx* h, const hkv_cache_desc* c) {
  if (!h || !c) return HKV_ERR_NULL_POINTER;
  if (!c->hot || !c->tail || !c->cold || !c->scales || !c->headers || !c->seq_len_dev || !c->seq_len_host)
    return HKV_ERR_NULL_POINTER;
  if (c->batch < 1 || c->max_blocks_per_seq < 0 || c->num_phys_blocks < 0) return HKV_ERR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(c->hot) % 512 != 0) return HKV_ERR_ALIGNMENT;
  const void* ptrs[] = {c->tail, c->cold, c->scales, c->headers, c->seq_len_dev};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return HKV_ERR_ALIGNMENT;
  for (int b = 0; b < c->batch; ++b)
    if (c->seq_len_host[b] < 0) return HKV_ERR_INVALID_VALUE;
  return HKV_OK;
}

hkv::CacheView view_of(const hkv_ctx* h, const hkv_cache_desc* c) {
  hkv::CacheView v;
  v.B = c->batch;
  v.H = h->H;
  v.D = h->D;
  v.T = h->T;
  v.S = h->S;
  v.bits = h->bits;
  v.max_blocks = c->max_blocks_per_seq;
  v.num_phys = c->num_phys_blocks;
  v.hot = static_cast<_Float16*>(c->hot);
  v.tail = static_cast<_Float16*>(c->tail);
  v.cold = c->cold;
  v.scales = c->scales;
  v.headers = c->headers;
  v.seq_len = c->seq_len_dev;
  v.quant_err = c->quant_err;
  v.entropy = c->entropy;
  return v;
}

// Decode workspace: partials [B][H][nsplit + 1][G][D + 2] fp32, then one arrival
// counter per (sequence, kv-head).
size_t partials_bytes(const hkv_ctx* h, const hkv_cache_desc* c, int G, int k_sel) {
  const int64_t bh = static_cast<int64_t>(c->batch) * h->H;
  int ns = max_splits(bh, std::max<int64_t>(1, c->max_blocks_per_seq));
  if (h->force_splits > 0) ns = std::max(ns, std::min(h->force_splits, kMaxSplits));
  if (k_sel > 0) ns = std::max(ns, plan_sparse(k_sel).nsplit);
  // ns cold splits + the hot zone (+ the tail block of a fused append)
  return static_cast<size_t>(bh) * (ns + 2) * G * (h->D + hkv::kRecHead) * sizeof(float);
}

// counters: [B*H] arrivals per (sequence, kv-head), [B] per sequence (fused append + decode), then
// (256-byte aligned) unit claims per (sequence, kv-head), one per 256 bytes: the claims of a
// (sequence, kv-head) are a steady stream of atomics, and counters that share a cache line would
// serialise each other's
size_t claim_offset(const hkv_cache_desc* c, int H) {
  return align_up(static_cast<size_t>(c->batch) * (H + 1) * sizeof(unsigned), 256);
}
size_t counters_bytes(const hkv_cache_desc* c, int H) {
  return claim_offset(c, H) + static_cast<size_t>(c->batch) * H * hkv::kClaimStride * sizeof(unsigned);
}
unsigned* claim_counters(void* workspace, const hkv_cache_desc* c, int H) {
  return reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + claim_offset(c, H));
}

// Top-K workspace after the counters: window probabilities [B][H][max_blocks * S] fp32, window tops
// [B][H][max_blocks] (kWinTop keys of 4 bytes) and their lanes [B][H][max_blocks] (one byte per
// top), every area 256-byte aligned.
struct TopkLayout {
  size_t wtop_off, wlane_off, bytes;  // offsets from the start of the probabilities
};
TopkLayout topk_layout(const hkv_ctx* h, const hkv_cache_desc* c) {
  const size_t bh = static_cast<size_t>(c->batch) * h->H;
  const size_t mb = static_cast<size_t>(std::max(0, c->max_blocks_per_seq));
  TopkLayout l;
  l.wtop_off = align_up(bh * mb * h->S * sizeof(float), 256);
  l.wlane_off = l.wtop_off + align_up(bh * mb * 4 * hkv::kWinTop, 256);
  l.bytes = l.wlane_off + bh * mb * hkv::kWinTop;
  return l;
}
size_t topk_bytes(const hkv_ctx* h, const hkv_cache_desc* c) { return topk_layout(h, c).bytes; }

LaunchCtx make_ctx(hkv_ctx* h, hipStream_t s, int kind) {
  LaunchCtx ctx{s, nullptr, nullptr};
  if (!h->timing) return ctx;
  hipEvent_t ev[2];
  for (hipEvent_t& e : ev) {
    if (!h->free_events.empty()) {
      e = h->free_events.back();
      h->free_events.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      return ctx;  // timing degrades to "not recorded", the launch still happens
    }
  }
  ctx.start = ev[0];
  ctx.stop = ev[1];
  h->pending.push_back({kind, ev[0], ev[1]});
  return ctx;
}

thread_local char g_detail[256] = "";

// Map a HIP failure to HKV_ERR_HIP and remember what failed for hkv_last_error_detail.
hkv_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return HKV_OK;
  snprintf(g_detail, sizeof(g_detail), "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
  return HKV_ERR_HIP;
}

// hkv_decode_attn and hkv_decode_attn_noalloc.  With `scratch` the workspace is the library's fixed
// device array on the current device (set up after every validation, before the launch) instead of
// the caller's buffer.
hkv_status decode_impl(hkv_ctx* h, const hkv_cache_desc* c, const void* q, int n_q_heads, const int32_t* sel_idx,
                       int k_sel, void* out, float* lse, void* workspace, size_t ws_bytes, hipStream_t stream,
                       bool scratch) {
  hkv_status st = check_desc(h, c);
  if (st != HKV_OK) return st;
  if (!q || !out) return HKV_ERR_NULL_POINTER;
  if (n_q_heads < 1 || n_q_heads % h->H != 0) return HKV_ERR_INVALID_VALUE;
  const int G = n_q_heads / h->H;
  if (sel_idx && (k_sel < 1 || k_sel > hkv::kMaxTopK)) return HKV_ERR_INVALID_VALUE;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HKV_ERR_UNSUPPORTED;
  int64_t units_max = 1;
  std::vector<int64_t> units(c->batch);
  for (int b = 0; b < c->batch; ++b) {
    const int n = c->seq_len_host[b];
    if (n == 0) return HKV_ERR_INVALID_VALUE;
    const int64_t nblk = cold_blocks(n, h->T, h->S);
    units[b] = nblk;
    if (!sel_idx) units_max = std::max(units_max, nblk);
  }
  size_t need = 0;
  if (hkv_workspace_bytes(h, c, n_q_heads, sel_idx ? k_sel : 0, &need) != HKV_OK) return HKV_ERR_INVALID_VALUE;
  // workspace layout: counters first, then the partials (for the fixed scratch: at a fixed offset)
  const size_t ctr_bytes = align_up(counters_bytes(c, h->H), 256);
  if (scratch) {
    if (ctr_bytes > hkv::kScratchCounterBytes ||
        align_up(partials_bytes(h, c, G, sel_idx ? k_sel : 0), 256) > hkv::kScratchBytes - hkv::kScratchCounterBytes)
      return HKV_ERR_WORKSPACE;
  } else if (!workspace || ws_bytes < need) {
    return HKV_ERR_WORKSPACE;
  }
  if ((!scratch && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) || reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return HKV_ERR_ALIGNMENT;
  uint16_t order[hkv::kOrderTableMax];
  if (h->timing) {  // the call's last host allocation, before its first HIP call
    h->pending.reserve(h->pending.size() + 1);
    h->free_events.reserve(h->free_events.size() + 2);
  }
  if (scratch) {
    const hipError_t e = hkv::scratch_for_device(stream, &workspace);
    if (e != hipSuccess) return hip_status(e, "hkv_decode_attn_noalloc scratch set-up");
  }

  hkv::DecodeParams p{};
  p.c = view_of(h, c);
  p.stamps = h->stamps;
  p.stamp_wgs = static_cast<int>(std::min<size_t>(h->stamp_wgs, INT32_MAX));
  p.G = G;
  p.q = static_cast<const _Float16*>(q);
  p.sel = sel_idx;
  p.k_sel = sel_idx ? k_sel : 0;
  p.counters = static_cast<unsigned*>(workspace);
  p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + (scratch ? hkv::kScratchCounterBytes : ctr_bytes));
  const SplitPlan sp = sel_idx ? plan_sparse(k_sel)
                      : h->force_splits > 0 ? forced_plan(units_max, h->force_splits)
                                            : stats_plan(c, dense_plan(h, static_cast<int64_t>(c->batch) * h->H, units_max,
                                                                       units_sum(units) * h->H, 1), units_max);
  p.nsplit = sp.nsplit;
  p.nparts = sp.nsplit + 1;
  p.units_per_split = sp.per_split;
  p.wg_order = sp.wg_order;
  p.work = (!sel_idx && sp.claim) ? claim_counters(workspace, c, h->H) : nullptr;
  p.k_new = p.v_new = nullptr;  // (before the order table: it counts the workgroups from them)
  const bool ordered = !sel_idx && sp.batch && order_by_work(p, units, sp.per_split, order);
  if (ordered) p.wg_order = hkv::kOrderTable;
  p.qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->D)));
  p.out = static_cast<_Float16*>(out);
  p.lse = lse;
  p.seq_counters = nullptr;
  p.store_units_base = nullptr;
  p.store_scales = nullptr;
  p.store_counts = nullptr;
  p.store_units = 0;
  LaunchCtx a = make_ctx(h, stream, sel_idx ? HKV_KERNEL_DECODE_SPARSE : HKV_KERNEL_DECODE);
  return hip_status(hkv::launch_decode(p, a, ordered ? order : nullptr),
                    scratch ? "hkv_decode_attn_noalloc launch" : "hkv_decode_attn launch");
}

// Runs an entry point's body; a failed host allocation (std::bad_alloc, or a
// length error from a huge count) becomes HKV_ERR_OUT_OF_MEMORY, so no C++
// exception crosses the C ABI.  Every body validates and allocates before its
// first HIP call, so nothing has been launched when this status is returned.
template <typename F>
hkv_status guarded(F&& body) noexcept {
  try {
    return body();
  } catch (...) {
    return HKV_ERR_OUT_OF_MEMORY;
  }
}

}  // namespace

extern "C" {

hkv_status hkv_create(int n_kv_heads, int head_dim, int hot_tokens, int block_size, int quant_bits,
                      hkv_handle* out) {
  if (!out) return HKV_ERR_NULL_POINTER;
  *out = nullptr;
  if (n_kv_heads < 1 || head_dim < 1) return HKV_ERR_INVALID_VALUE;
  if (!valid_protocol(hot_tokens, block_size)) return HKV_ERR_INVALID_VALUE;
  if (quant_bits != 0 && quant_bits != 4 && quant_bits != 8) return HKV_ERR_INVALID_VALUE;
  if (block_size != hkv::kBlockSize || (head_dim != 64 && head_dim != 128)) return HKV_ERR_UNSUPPORTED;
  hkv_ctx* h = new (std::nothrow) hkv_ctx;
  if (!h) return HKV_ERR_OUT_OF_MEMORY;
  h->H = n_kv_heads;
  h->D = head_dim;
  h->T = hot_tokens;
  h->S = block_size;
  h->bits = quant_bits;
  *out = h;
  return HKV_OK;
}

hkv_status hkv_destroy(hkv_handle h) {
  if (!h) return HKV_OK;
  for (auto& p : h->pending) {
    (void)hipEventSynchronize(p.stop);
    (void)hipEventDestroy(p.start);
    (void)hipEventDestroy(p.stop);
  }
  for (hipEvent_t e : h->free_events) (void)hipEventDestroy(e);
  delete h;
  return HKV_OK;
}

hkv_status hkv_cache_sizes(hkv_handle h, int batch, int64_t max_tokens_per_seq, int64_t num_phys_blocks,
                           hkv_cache_sizes_t* out) {
  if (!h || !out) return HKV_ERR_NULL_POINTER;
  if (batch < 1 || max_tokens_per_seq < 0 || num_phys_blocks < 0) return HKV_ERR_INVALID_VALUE;
  const int64_t mb = cold_blocks(max_tokens_per_seq, h->T, h->S);
  if (mb > INT32_MAX) return HKV_ERR_INVALID_VALUE;
  const int64_t P = num_phys_blocks ? num_phys_blocks : mb * batch;
  if (P > INT32_MAX) return HKV_ERR_INVALID_VALUE;
  out->hot = static_cast<size_t>(batch) * h->H * h->T * 2 * h->D * 2;
  out->tail = static_cast<size_t>(batch) * h->H * 2 * h->S * h->D * 2;
  out->cold = static_cast<size_t>(P) * h->H * 2 * tile_bytes(h);
  out->scales = static_cast<size_t>(P) * h->H * 2 * sizeof(float);
  out->headers = static_cast<size_t>(batch) * mb * sizeof(hkv_block_header);
  out->seq_len = static_cast<size_t>(batch) * sizeof(int32_t);
  out->max_blocks_per_seq = static_cast<int32_t>(mb);
  out->num_phys_blocks = static_cast<int32_t>(P);
  return HKV_OK;
}

hkv_status hkv_sizes(hkv_handle h, int batch, int max_tokens_per_seq, int num_phys_blocks, size_t bytes_out[6]) {
  if (!h || !bytes_out) return HKV_ERR_NULL_POINTER;
  hkv_cache_sizes_t s;
  const hkv_status st = hkv_cache_sizes(h, batch, max_tokens_per_seq, num_phys_blocks, &s);
  if (st != HKV_OK) return st;
  bytes_out[0] = s.hot;
  bytes_out[1] = s.tail;
  bytes_out[2] = s.cold;
  bytes_out[3] = s.scales;
  bytes_out[4] = s.headers;
  bytes_out[5] = s.seq_len;
  return HKV_OK;
}

hkv_status hkv_header_table_bytes(int hot_tokens, int block_size, int64_t total_tokens, int64_t* n_blocks,
                                  size_t* bytes) {
  if (!n_blocks || !bytes) return HKV_ERR_NULL_POINTER;
  if (!valid_protocol(hot_tokens, block_size) || total_tokens < 0) return HKV_ERR_INVALID_VALUE;
  *n_blocks = cold_blocks(total_tokens, hot_tokens, block_size);
  *bytes = static_cast<size_t>(*n_blocks) * sizeof(hkv_block_header);
  return HKV_OK;
}

hkv_status hkv_workspace_bytes(hkv_handle h, const hkv_cache_desc* c, int n_q_heads, int k_sel, size_t* bytes) {
  if (!h || !c || !bytes) return HKV_ERR_NULL_POINTER;
  if (c->batch < 1 || c->max_blocks_per_seq < 0) return HKV_ERR_INVALID_VALUE;
  if (n_q_heads < 1 || n_q_heads % h->H != 0) return HKV_ERR_INVALID_VALUE;
  if (k_sel < 0 || k_sel > hkv::kMaxTopK) return HKV_ERR_INVALID_VALUE;
  const int G = n_q_heads / h->H;
  // the counters sit at the front so that their offset does not depend on the state
  size_t ws = align_up(counters_bytes(c, h->H), 256) + align_up(partials_bytes(h, c, G, k_sel), 256);
  if (k_sel > 0) ws = std::max(ws, align_up(counters_bytes(c, h->H), 256) + align_up(topk_bytes(h, c), 256));
  *bytes = std::max<size_t>(ws, 256);
  return HKV_OK;
}

hkv_status hkv_append(hkv_handle h, const hkv_cache_desc* c, const void* k_new, const void* v_new,
                      const int32_t* n_new_host, int max_n_new, hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    hkv_status st = check_desc(h, c);
    if (st != HKV_OK) return st;
    if (!n_new_host) return HKV_ERR_NULL_POINTER;
    if (max_n_new < 0) return HKV_ERR_INVALID_VALUE;
    bool any = false;
    for (int b = 0; b < c->batch; ++b) {
      const int nn = n_new_host[b];
      if (nn < 0 || nn > max_n_new) return HKV_ERR_INVALID_VALUE;
      const int64_t n1 = static_cast<int64_t>(c->seq_len_host[b]) + nn;
      if (n1 > INT32_MAX) return HKV_ERR_CAPACITY;
      if (cold_blocks(n1, h->T, h->S) > c->max_blocks_per_seq) return HKV_ERR_CAPACITY;
      if (nn > 0) any = true;
    }
    if (!any) return HKV_OK;
    if (!k_new || !v_new) return HKV_ERR_NULL_POINTER;
    if (reinterpret_cast<uintptr_t>(k_new) % 16 != 0 || reinterpret_cast<uintptr_t>(v_new) % 16 != 0)
      return HKV_ERR_ALIGNMENT;

    if (h->timing) {  // every host allocation of the call happens here, before the first launch
      const size_t chunks = (static_cast<size_t>(c->batch) + hkv::kAppendChunk - 1) / hkv::kAppendChunk;
      h->pending.reserve(h->pending.size() + 2 * chunks);
      h->free_events.reserve(h->free_events.size() + 2 * chunks);
    }
    hkv::AppendParams p{};
    std::memset(&p, 0, sizeof(p));
    p.c = view_of(h, c);
    p.k_new = static_cast<const _Float16*>(k_new);
    p.v_new = static_cast<const _Float16*>(v_new);
    p.max_n_new = max_n_new;
    for (int b0 = 0; b0 < c->batch; b0 += hkv::kAppendChunk) {
      const int ns = std::min(hkv::kAppendChunk, c->batch - b0);
      int touched = 0;
      bool chunk_any = false;
      for (int i = 0; i < ns; ++i) {
        const int b = b0 + i;
        const int nn = n_new_host[b];
        p.n_new[i] = nn;
        p.n0[i] = c->seq_len_host[b];
        if (nn == 0) continue;
        chunk_any = true;
        const int64_t n0 = c->seq_len_host[b], n1 = n0 + nn;
        const int64_t cold0 = std::max<int64_t>(0, n0 - h->T), cold1 = std::max<int64_t>(0, n1 - h->T);
        if (cold1 > cold0) touched = std::max<int>(touched, static_cast<int>((cold1 + h->S - 1) / h->S - cold0 / h->S));
      }
      if (!chunk_any) continue;
      p.b0 = b0;
      p.n_seq = ns;
      p.touched_max = touched;
      p.single_pass = touched <= hkv::kSinglePassMaxBlocks ? 1 : 0;
      LaunchCtx qctx = make_ctx(h, stream, HKV_KERNEL_APPEND);
      LaunchCtx rctx = p.single_pass ? LaunchCtx{stream, nullptr, nullptr} : make_ctx(h, stream, HKV_KERNEL_APPEND_RING);
      if (touched == 0 && !p.single_pass && qctx.start) {  // nothing to quantise: release the unused event pair
        h->free_events.push_back(qctx.start);
        h->free_events.push_back(qctx.stop);
        h->pending.erase(h->pending.end() - 2);
        qctx.start = qctx.stop = nullptr;
      }
      hipError_t e = hkv::launch_append(p, qctx, rctx);
      if (e != hipSuccess) return hip_status(e, "hkv_append launch");
    }
    for (int b = 0; b < c->batch; ++b) c->seq_len_host[b] += n_new_host[b];
    return HKV_OK;
  });
}

hkv_status hkv_decode_attn(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads,
                           const int32_t* sel_idx, int k_sel, void* out, float* lse, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    return decode_impl(h, c, q, n_q_heads, sel_idx, k_sel, out, lse, workspace, ws_bytes, stream, false);
  });
}

hkv_status hkv_decode_attn_noalloc(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads,
                                   const int32_t* sel_idx, int k_sel, void* out, float* lse, hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    return decode_impl(h, c, q, n_q_heads, sel_idx, k_sel, out, lse, nullptr, 0, stream, true);
  });
}

hkv_status hkv_append_decode(hkv_handle h, const hkv_cache_desc* c, const void* k_new, const void* v_new,
                             const void* q, int n_q_heads, void* out, float* lse, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    hkv_status st = check_desc(h, c);
    if (st != HKV_OK) return st;
    if (!k_new || !v_new || !q || !out) return HKV_ERR_NULL_POINTER;
    if (n_q_heads < 1 || n_q_heads % h->H != 0) return HKV_ERR_INVALID_VALUE;
    const int G = n_q_heads / h->H;
    if (G != 1 && G != 2 && G != 4 && G != 8) return HKV_ERR_UNSUPPORTED;
    if (h->S != hkv::kBlockSize) return HKV_ERR_UNSUPPORTED;
    int64_t units_max = 1;
    std::vector<int64_t> units(c->batch);
    for (int b = 0; b < c->batch; ++b) {
      const int64_t n0 = c->seq_len_host[b];
      if (n0 < 0) return HKV_ERR_INVALID_VALUE;
      if (n0 + 1 > INT32_MAX) return HKV_ERR_CAPACITY;
      if (cold_blocks(n0 + 1, h->T, h->S) > c->max_blocks_per_seq) return HKV_ERR_CAPACITY;
      // cold units of the decode: the full blocks before the one the appended token spills into
      units[b] = std::max<int64_t>(0, n0 - h->T) / h->S;
      units_max = std::max<int64_t>(units_max, units[b]);
    }
    size_t need = 0;
    if (hkv_workspace_bytes(h, c, n_q_heads, 0, &need) != HKV_OK) return HKV_ERR_INVALID_VALUE;
    if (!workspace || ws_bytes < need) return HKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(k_new) % 16 != 0 || reinterpret_cast<uintptr_t>(v_new) % 16 != 0)
      return HKV_ERR_ALIGNMENT;

    hkv::DecodeParams p{};
    p.c = view_of(h, c);
    p.stamps = h->stamps;
    p.stamp_wgs = static_cast<int>(std::min<size_t>(h->stamp_wgs, INT32_MAX));
    p.G = G;
    p.q = static_cast<const _Float16*>(q);
    p.sel = nullptr;
    p.k_sel = 0;
    p.counters = static_cast<unsigned*>(workspace);
    p.seq_counters = p.counters + static_cast<size_t>(c->batch) * h->H;
    p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(counters_bytes(c, h->H), 256));
    const SplitPlan sp = h->force_splits > 0 ? forced_plan(units_max, h->force_splits)
                                             : stats_plan(c, dense_plan(h, static_cast<int64_t>(c->batch) * h->H, units_max,
                                                                        units_sum(units) * h->H, 1), units_max);
    p.nsplit = sp.nsplit;
    p.nparts = sp.nsplit + 2;
    p.units_per_split = sp.per_split;
    p.wg_order = sp.wg_order;
    p.work = sp.claim ? claim_counters(workspace, c, h->H) : nullptr;
    p.k_new = static_cast<const _Float16*>(k_new);  // (before the order table: it counts the workgroups from them)
    p.v_new = static_cast<const _Float16*>(v_new);
    // lengths before the append from the host mirror, in the launch arguments (up to kFusedLenMax sequences)
    p.host_lens = c->batch <= hkv::kFusedLenMax ? 1 : 0;
    p.n0_host = c->seq_len_host;
    uint16_t order[hkv::kOrderTableMax];
    const bool ordered = sp.batch && order_by_work(p, units, sp.per_split, order);
    if (ordered) p.wg_order = hkv::kOrderTable;
    p.qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->D)));
    p.out = static_cast<_Float16*>(out);
    p.lse = lse;
    p.store_units_base = nullptr;
    p.store_scales = nullptr;
    p.store_counts = nullptr;
    p.store_units = 0;
    LaunchCtx a = make_ctx(h, stream, HKV_KERNEL_APPEND_DECODE);
    const hkv_status r = hip_status(hkv::launch_decode(p, a, ordered ? order : nullptr), "hkv_append_decode launch");
    if (r != HKV_OK) return r;
    for (int b = 0; b < c->batch; ++b) c->seq_len_host[b] += 1;
    return HKV_OK;
  });
}

hkv_status hkv_sparse_store_bytes(hkv_handle h, int batch, int k_sel, size_t* bytes) {
  if (!h || !bytes) return HKV_ERR_NULL_POINTER;
  if (batch < 1 || k_sel < 1 || k_sel > hkv::kMaxTopK) return HKV_ERR_INVALID_VALUE;
  *bytes = store_layout(h, batch, k_sel).bytes;
  return HKV_OK;
}

hkv_status hkv_sparse_compact(hkv_handle h, const hkv_cache_desc* c, const int32_t* sel_idx, int k_sel, void* store,
                              size_t store_bytes, hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    hkv_status st = check_desc(h, c);
    if (st != HKV_OK) return st;
    if (!sel_idx || !store) return HKV_ERR_NULL_POINTER;
    if (k_sel < 1 || k_sel > hkv::kMaxTopK) return HKV_ERR_INVALID_VALUE;
    if (h->S != hkv::kBlockSize) return HKV_ERR_UNSUPPORTED;
    const StoreLayout l = store_layout(h, c->batch, k_sel);
    if (store_bytes < l.bytes) return HKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(store) % 256 != 0 || reinterpret_cast<uintptr_t>(sel_idx) % 4 != 0)
      return HKV_ERR_ALIGNMENT;
    if (h->timing) {
      h->pending.reserve(h->pending.size() + 1);
      h->free_events.reserve(h->free_events.size() + 2);
    }
    hkv::CompactParams p{};
    p.c = view_of(h, c);
    p.sel = sel_idx;
    p.k_sel = k_sel;
    p.units = l.units;
    p.counts = static_cast<int32_t*>(store);
    p.scales = reinterpret_cast<float2*>(static_cast<char*>(store) + l.scales_off);
    p.units_base = static_cast<int8_t*>(store) + l.units_off;
    LaunchCtx a = make_ctx(h, stream, HKV_KERNEL_SPARSE_COMPACT);
    return hip_status(hkv::launch_compact(p, a), "hkv_sparse_compact launch");
  });
}

hkv_status hkv_decode_attn_compact(hkv_handle h, const hkv_cache_desc* c, const void* store, int k_sel, const void* q,
                                   int n_q_heads, void* out, float* lse, void* workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    hkv_status st = check_desc(h, c);
    if (st != HKV_OK) return st;
    if (!store || !q || !out) return HKV_ERR_NULL_POINTER;
    if (n_q_heads < 1 || n_q_heads % h->H != 0) return HKV_ERR_INVALID_VALUE;
    const int G = n_q_heads / h->H;
    if (k_sel < 1 || k_sel > hkv::kMaxTopK) return HKV_ERR_INVALID_VALUE;
    if (G != 1 && G != 2 && G != 4 && G != 8) return HKV_ERR_UNSUPPORTED;
    if (h->S != hkv::kBlockSize) return HKV_ERR_UNSUPPORTED;
    for (int b = 0; b < c->batch; ++b)
      if (c->seq_len_host[b] == 0) return HKV_ERR_INVALID_VALUE;
    size_t need = 0;
    if (hkv_workspace_bytes(h, c, n_q_heads, k_sel, &need) != HKV_OK) return HKV_ERR_INVALID_VALUE;
    if (!workspace || ws_bytes < need) return HKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(store) % 256 != 0)
      return HKV_ERR_ALIGNMENT;
    if (h->timing) {
      h->pending.reserve(h->pending.size() + 1);
      h->free_events.reserve(h->free_events.size() + 2);
    }
    const StoreLayout l = store_layout(h, c->batch, k_sel);
    hkv::DecodeParams p{};
    p.c = view_of(h, c);
    p.stamps = h->stamps;
    p.stamp_wgs = static_cast<int>(std::min<size_t>(h->stamp_wgs, INT32_MAX));
    p.G = G;
    p.q = static_cast<const _Float16*>(q);
    p.sel = nullptr;
    p.k_sel = k_sel;
    p.counters = static_cast<unsigned*>(workspace);
    p.partials = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(counters_bytes(c, h->H), 256));
    // one unit of 64 stored tokens per wave: every unit of the call is in flight at once
    p.units_per_split = hkv::kWaves;
    p.nsplit = (l.units + hkv::kWaves - 1) / hkv::kWaves;
    p.nparts = p.nsplit + 1;
    p.wg_order = hkv::kOrderPlain;
    p.work = nullptr;
    p.qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(h->D)));
    p.out = static_cast<_Float16*>(out);
    p.lse = lse;
    p.k_new = p.v_new = nullptr;
    p.seq_counters = nullptr;
    p.store_counts = static_cast<const int32_t*>(store);
    p.store_scales = reinterpret_cast<const float2*>(static_cast<const char*>(store) + l.scales_off);
    p.store_units_base = static_cast<const int8_t*>(store) + l.units_off;
    p.store_units = l.units;
    LaunchCtx a = make_ctx(h, stream, HKV_KERNEL_DECODE_COMPACT);
    return hip_status(hkv::launch_decode(p, a, nullptr), "hkv_decode_attn_compact launch");
  });
}

hkv_status hkv_topk_select(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads, int k,
                           int32_t* out_idx, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return guarded([&]() -> hkv_status {
    hkv_status st = check_desc(h, c);
    if (st != HKV_OK) return st;
    if (!q || !out_idx) return HKV_ERR_NULL_POINTER;
    if (n_q_heads < 1 || n_q_heads % h->H != 0) return HKV_ERR_INVALID_VALUE;
    if (k < 1 || k > hkv::kMaxTopK) return HKV_ERR_INVALID_VALUE;
    const int G = n_q_heads / h->H;
    if (G != 1 && G != 2 && G != 4 && G != 8) return HKV_ERR_UNSUPPORTED;
    if (h->S != hkv::kBlockSize) return HKV_ERR_UNSUPPORTED;
    size_t need = 0;
    if (hkv_workspace_bytes(h, c, n_q_heads, k, &need) != HKV_OK) return HKV_ERR_INVALID_VALUE;
    if (!workspace || ws_bytes < need) return HKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0)
      return HKV_ERR_ALIGNMENT;
    int64_t blk_max = 1;
    for (int b = 0; b < c->batch; ++b) blk_max = std::max(blk_max, cold_blocks(c->seq_len_host[b], h->T, h->S));

    const TopkLayout tl = topk_layout(h, c);
    hkv::TopkParams p{};
    p.c = view_of(h, c);
    p.G = G;
    p.q = static_cast<const _Float16*>(q);
    char* const area = static_cast<char*>(workspace) + align_up(counters_bytes(c, h->H), 256);
    p.prob = reinterpret_cast<float*>(area);
    p.wtop = reinterpret_cast<uint4*>(area + tl.wtop_off);
    p.wlane = reinterpret_cast<uint32_t*>(area + tl.wlane_off);
    // the score kernel holds at most 64 VGPRs per lane (D = 128, G <= 4), so 8 of its workgroups fit a
    // CU: twice the decode's grid; its claim plans take 4 per CU (32768-token workload, measured:
    // static splits 98.6 us, claims on 512 / 1024 / 2048 workgroups 98.5 / 91.3 / 92.7 us)
    const SplitPlan sp = plan_splits(static_cast<int64_t>(c->batch) * h->H, blk_max, 1, 2 * kTargetWorkgroups,
                                     kTopkClaimTargetWorkgroups);
    p.nsplit = sp.nsplit;
    p.units_per_split = sp.per_split;
    p.wg_order = sp.wg_order;
    p.work = sp.claim ? claim_counters(workspace, c, h->H) : nullptr;
    p.k = k;
    p.out_idx = out_idx;
    LaunchCtx a = make_ctx(h, stream, HKV_KERNEL_TOPK_SCORE);
    LaunchCtx b = make_ctx(h, stream, HKV_KERNEL_TOPK_SELECT);
    return hip_status(hkv::launch_topk(p, a, b), "hkv_topk_select launch");
  });
}

hkv_status hkv_read_probe(const void* src, size_t bytes, int workgroups, int threads, uint32_t* sink,
                          hipStream_t stream) {
  if (!src || !sink) return HKV_ERR_NULL_POINTER;
  if (workgroups < 1 || threads < 64 || threads > 1024 || threads % 64 != 0 || bytes % 16 != 0)
    return HKV_ERR_INVALID_VALUE;
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return HKV_ERR_ALIGNMENT;
  return hip_status(hkv::launch_read_probe(src, bytes, workgroups, threads, sink, LaunchCtx{stream, nullptr, nullptr}),
                    "hkv_read_probe launch");
}

const char* hkv_last_error_detail(void) { return g_detail; }

const char* hkv_status_string(hkv_status st) {
  switch (st) {
    case HKV_OK: return "ok";
    case HKV_ERR_INVALID_VALUE: return "invalid value";
    case HKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case HKV_ERR_NULL_POINTER: return "null pointer";
    case HKV_ERR_CAPACITY: return "cache capacity exceeded";
    case HKV_ERR_WORKSPACE: return "workspace missing or too small";
    case HKV_ERR_HIP: return "HIP runtime error";
    case HKV_ERR_ALIGNMENT: return "misaligned buffer";
    case HKV_ERR_OUT_OF_MEMORY: return "out of host memory";
  }
  return "unknown status";
}

hkv_status hkv_plan_override(hkv_handle h, int nsplit, int claim_workgroups) {
  if (!h) return HKV_ERR_NULL_POINTER;
  if (nsplit < 0 || nsplit > kMaxSplits || claim_workgroups < 0 || claim_workgroups > 65536)
    return HKV_ERR_INVALID_VALUE;
  h->force_splits = nsplit;
  h->claim_workgroups = claim_workgroups;
  return HKV_OK;
}

hkv_status hkv_phase_stamps(hkv_handle h, uint64_t* buf, size_t bytes) {
  if (!h) return HKV_ERR_NULL_POINTER;
  if (buf && reinterpret_cast<uintptr_t>(buf) % 8 != 0) return HKV_ERR_ALIGNMENT;
  h->stamps = reinterpret_cast<unsigned long long*>(buf);
  h->stamp_wgs = buf ? bytes / (8 * sizeof(uint64_t)) : 0;
  return HKV_OK;
}

hkv_status hkv_timing_enable(hkv_handle h, int enable) {
  if (!h) return HKV_ERR_NULL_POINTER;
  h->timing = enable != 0;
  return HKV_OK;
}

hkv_status hkv_timing_read(hkv_handle h, int kind, double* total_ms, int64_t* count, int reset) {
  return guarded([&]() -> hkv_status {
    if (!h || !total_ms || !count) return HKV_ERR_NULL_POINTER;
    if (kind < 0 || kind >= HKV_KERNEL_KINDS) return HKV_ERR_INVALID_VALUE;
    std::vector<hkv_ctx::Pending> keep;
    keep.reserve(h->pending.size());
    for (auto& p : h->pending) {
      if (p.kind != kind) {
        keep.push_back(p);
        continue;
      }
      hipError_t e = hipEventSynchronize(p.stop);
      if (e != hipSuccess) return hip_status(e, "hkv_timing_read sync");
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, p.start, p.stop);
      if (e != hipSuccess) return hip_status(e, "hkv_timing_read elapsed");
      h->total_ms[kind] += ms;
      h->count[kind] += 1;
      h->free_events.push_back(p.start);
      h->free_events.push_back(p.stop);
    }
    h->pending.swap(keep);
    *total_ms = h->total_ms[kind];
    *count = h->count[kind];
    if (reset) {
      h->total_ms[kind] = 0.0;
      h->count[kind] = 0;
    }
    return HKV_OK;
  });
}

}  // extern "C"
