// Internal launch interface of libhkv: parameter blocks passed by value to the
// gfx950 kernels and the host-side launch wrappers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkv.h"

namespace hkv {

constexpr int kBlockSize = 64;      // tokens per cold block (the only built value)
constexpr int kThreads = 256;       // 4 wave64 per workgroup for the streaming kernels
constexpr int kWaves = kThreads / 64;
constexpr int kAppendChunk = 256;   // sequences whose append counts travel in one kernel-argument block
constexpr int kSinglePassMaxBlocks = 2;  // appends touching at most this many blocks per sequence use one launch
constexpr int kMaxTopK = 512;       // fixed top-K budget of the sparse path
constexpr int kSparseUnit = 16;     // selected tokens per wave unit of the sparse decode
constexpr int kOrderPlain = 0, kOrderSplitMajor = 2, kOrderTable = 3;  // workgroup orders (see wg_coord)
constexpr int kOrderTableMax = 512;  // (sequence, part) groups a table order can list
constexpr int kClaimUnits = 16;     // plans with splits of at least this many units claim them dynamically
constexpr int kClaimStride = 64;    // claim counters 256 bytes apart: one cache line each
constexpr int kMaxSplits = 128;     // cold splits per (sequence, kv-head) at most
constexpr int kRecHead = 4;         // floats before acc[D] in a partial record: m, l, z (sum of w * logit), 0
// Fixed device scratch of hkv_decode_attn_noalloc, per GPU: the counters of every call live in the
// first kScratchCounterBytes, the split partials after them, so the partials of one call never land
// on the counters of another (every call leaves all of its counters at zero).
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchCounterBytes = size_t(4) << 20;

// Per-launch timing: when start/stop are non-null the dispatch records them.
struct LaunchCtx {
  hipStream_t stream;
  hipEvent_t start;
  hipEvent_t stop;
};

struct CacheView {
  int B, H, D, T, S;
  int bits;            // cold-tile format: 8- or 4-bit codes, 0 = fp16 values
  int max_blocks, num_phys;
  _Float16* hot;       // [B][H][T][2][D]
  _Float16* tail;      // [B][H][2][S][D]
  int8_t* cold;        // [P][H][2][tile bytes]
  float* scales;       // [P][H][2]
  hkv_block_header* headers;  // [B][max_blocks]
  int32_t* seq_len;    // [B]
  float* quant_err;    // [P][H][2] debug statistic or nullptr
  float* entropy;      // [B][H*G] debug statistic or nullptr
};

struct AppendParams {
  CacheView c;
  const _Float16* k_new;   // [B][max_n_new][H][D]
  const _Float16* v_new;
  int max_n_new;
  int b0;                  // first sequence of this launch
  int n_seq;               // sequences in this launch (<= kAppendChunk)
  int touched_max;         // grid extent over touched cold blocks per sequence
  int single_pass;         // 1: append_step_kernel (lengths from n0[]), 0: two-pass kernels
  int32_t n_new[kAppendChunk];
  int32_t n0[kAppendChunk];  // cached length before the append (host mirror)
};

struct DecodeParams {
  CacheView c;
  int G;                   // query heads per kv-head
  const _Float16* q;       // [B][H*G][D]
  const int32_t* sel;      // sparse mode: [B][H][k_sel]; nullptr for dense
  int k_sel;
  float* partials;         // [B][H][nparts][G][D + 4]  (m in log2 units, l, z, 0, acc[D]); then hot zone, tail block
  unsigned* counters;      // [B*H] arrival counters, zero between calls
  int nsplit;              // cold splits per (sequence, kv-head)
  int nparts;              // partial records per (sequence, kv-head): nsplit + 1 (hot zone), + 1 more fused
                           // (the fused append's workgroup writes the last two: see grid_parts)
  int units_per_split;     // units handled per split (multiple of kWaves)
  int wg_order;            // kOrderPlain / kOrderSplitMajor / kOrderTable (see wg_coord)
  int order_groups;        // kOrderTable: (sequence, part) groups the table lists (the grid is H x groups)
  unsigned* work;          // [B*H][kClaimStride] unit-claim counters (dense walk), zero between calls; nullptr: static
  float qscale;            // log2(e) / sqrt(D)
  _Float16* out;           // [B][H*G][D]
  float* lse;              // [B][H*G] or nullptr
  // fused single-token append (hkv_append_decode); nullptr for a plain decode
  const _Float16* k_new;   // [B][H][D]
  const _Float16* v_new;   // [B][H][D]
  unsigned* seq_counters;  // [B] merged-head counters, zero between calls
  // fused step of at most kFusedLenMax sequences: the lengths before the append travel in the launch
  // arguments (DecodeParamsFused::n0, DecodeParamsOrdered::n0), so no workgroup reads seq_len and
  // one plain store per sequence publishes the new length.  0: seq_len is read, and the last of the
  // H merges of a sequence publishes it (seq_counters).
  int host_lens;
  const int32_t* n0_host;  // host side only: the host mirror the launch copies into n0 (never read on the GPU)
  // decode over a compacted sparse store (CompactParams layout); store_units_base nullptr otherwise
  const int8_t* store_units_base;
  const float2* store_scales;
  const int32_t* store_counts;
  int store_units;
  // phase timestamps (hkv_phase_stamps): 8 x uint64 per workgroup, stamp_wgs workgroups; nullptr = off
  unsigned long long* stamps;
  int stamp_wgs;
};

// Compacted sparse store of a selection (see compact.hip): per (sequence, kv-head) `units` units of
// 64 tokens, each a K tile and a V tile in the cold-block chunk layouts.
struct CompactParams {
  CacheView c;
  const int32_t* sel;      // [B][H][k_sel]
  int k_sel;
  int units;               // units per (sequence, kv-head) = ceil(k_sel / 64)
  int32_t* counts;         // [B*H] stored tokens
  float2* scales;          // [B*H][units][64] (K scale, V scale) of each stored token
  int8_t* units_base;      // [B*H][units][2][tile bytes]
};

// Workgroups per (sequence, kv-head) of a decode launch: one per partial record, except that a fused
// append + decode's last workgroup attends the hot window and the tail block, two records.
__host__ __device__ inline int grid_parts(const DecodeParams& p) { return p.nparts - (p.k_new ? 1 : 0); }

// Sequences whose lengths a fused step takes from its launch arguments (see DecodeParams::host_lens).
constexpr int kFusedLenMax = 256;

// Arguments of the fused one-token append + decode in the plain, split-major and claim orders.
struct DecodeParamsFused {
  DecodeParams p;
  int32_t n0[kFusedLenMax];  // the cached length of each sequence before the append (p.host_lens)
};

// Arguments of the table-ordered decode launch (batch plans): the (sequence << 7 | part) groups
// of the grid in dispatch order, [B * grid_parts] entries used; and, for a fused step, the lengths.
struct DecodeParamsOrdered {
  DecodeParams p;
  uint16_t order[kOrderTableMax];
  int32_t n0[kFusedLenMax];  // the cached length of each sequence before the append (p.host_lens)
};

// Cold splits of one (sequence, kv-head) in a table-ordered launch: enough splits of units_per_split
// units for its own unit count (at least one, at most nsplit); the host's table lists only these
// (device and host compute it from the same unit count).  Other launches use all nsplit.
__host__ __device__ inline int table_splits(int nsplit, int units_per_split, int64_t units) {
  const int64_t n = (units + units_per_split - 1) / units_per_split;
  return static_cast<int>(n < 1 ? 1 : (n > nsplit ? nsplit : n));
}

// Top-K selection (topk.hip): the score kernel keeps the kWinTop largest keys of every window and
// their lanes; one kSelThreads-thread workgroup per row selects from those (rows of up to
// kTopsWindows windows), staging at most kFinalKeys candidates.
constexpr int kWinTop = 4;
constexpr int kSelThreads = 512;
constexpr int kFinalKeys = 4096;
constexpr int kDirectKeys = 8192;    // rows of at most this many keys are selected from the row itself
constexpr int kTopsWindows = 2048;   // rows of up to 131072 keys are selected from their window tops

struct TopkParams {
  CacheView c;
  int G;
  const _Float16* q;       // [B][H*G][D]
  float* prob;             // [B][H][max_blocks*S] window probabilities
  uint4* wtop;             // [B][H][max_blocks] each window's kWinTop largest keys, in lane order
                           //   (fp32 bits + 1; 0 = none)
  uint32_t* wlane;         // [B][H][max_blocks] their lanes in the window, 8 bits each
  int nsplit;
  int units_per_split;
  int wg_order;            // kOrderPlain / kOrderSplitMajor / kOrderTable (see wg_coord)
  unsigned* work;          // [B*H][kClaimStride] unit-claim counters of the score walk; nullptr: static walk
  int k;
  int32_t* out_idx;        // [B][H][k]
};

hipError_t launch_append(const AppendParams& p, const LaunchCtx& quant_ctx, const LaunchCtx& ring_ctx);
// Decode launches of one (head_dim, group, cold-tile format) instance (decode_inst.hip).
template <int D, int G, int BITS>
hipError_t launch_decode_dgb(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order);

// Dispatch on (cold-tile format, head_dim, group) to the instances above (host code only: where the
// kernels' template definitions are visible, this body would instantiate every instance).
hipError_t launch_decode(const DecodeParams& p, const LaunchCtx& ctx, const uint16_t* order = nullptr);
hipError_t launch_topk(const TopkParams& p, const LaunchCtx& score_ctx, const LaunchCtx& sel_ctx);
// Device address of the fixed scratch array on the current device (set up on first use: address
// taken with hipGetSymbolAddress, array cleared on `stream`).
hipError_t scratch_for_device(hipStream_t stream, void** out);
hipError_t launch_compact(const CompactParams& p, const LaunchCtx& ctx);
hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, int threads, uint32_t* sink,
                             const LaunchCtx& ctx);

}  // namespace hkv
