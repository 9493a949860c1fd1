/*
 * hkv.h -- C ABI of libhkv: hybrid FP16-hot / INT8-cold KV cache and
 * single-token decode attention on AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by short title and section:
 *   "Hybrid KV Cache page": DeepSeek V4 hybrid KV Cache inference
 *       optimisation: hands-on analysis (tqpw.cn news 44343).
 *   "KV Cache reuse page": KV Cache reuse: the key to LLM-inference memory
 *       and throughput (yfxerp.com news 372023), HySparse part.
 *   "V4 architecture page": DeepSeek V4 architecture: MoE dynamic loading and
 *       hierarchical KV cache (xxmr.cn news 3419).
 *
 * The cache (Hybrid KV Cache page, 2.1 and 3.2): the most recent
 * `hot_tokens` tokens of every sequence stay in FP16 ("hot zone", K and V
 * interleaved per token); older tokens live in `block_size`-token cold blocks
 * stored as INT8 with one fp32 scale per (block, kv-head, K|V), reached
 * through a 16-byte block header holding the physical block id and the
 * valid-token count.  Quantisation: s = fl32(max|x| / 127), code =
 * clamp(rint(fl32(x / s)), -127, 127) with round-half-to-even; a partially
 * filled last block always holds the codes of its current valid tokens (its
 * FP16 originals are kept in a per-sequence tail shadow so that the block can
 * be re-quantised when its scale grows).
 *
 * Conventions for every entry point:
 *   - The caller owns every buffer and the stream.  Device buffers are passed
 *     as raw device pointers (e.g. from torch tensors); arrays documented as
 *     "host" are plain host memory read during the call.
 *   - All validation is host-side and synchronous and happens before any HIP
 *     call; on an error nothing is launched and no buffer is touched.  A
 *     failed host-side allocation inside the library (launch planning uses a
 *     few small host arrays) returns HKV_ERR_OUT_OF_MEMORY, also before any
 *     launch; no C++ exception ever leaves an entry point.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream);
 *     results are valid after the stream is synchronised.  Calls on the same
 *     cache must be ordered on one stream; different caches are independent.
 *   - A handle is immutable after hkv_create except for its optional timing
 *     state (hkv_timing_*); a handle must not be used from two host threads at
 *     once while timing is enabled.
 */
#ifndef HKV_H_
#define HKV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hkv_ctx* hkv_handle;

/* Status codes.  Invalid parameters are reported synchronously at the call,
 * the host-side counterpart of the launch-time CUDA_ERROR_INVALID_VALUE the
 * Hybrid KV Cache page (3.1, 5.1) describes for bad hot_tokens/block_size. */
typedef enum {
  HKV_OK = 0,
  HKV_ERR_INVALID_VALUE = -1, /* a parameter breaks the protocol rules or a shape/count is out of range */
  HKV_ERR_UNSUPPORTED = -2,   /* valid per the protocol but not built (see hkv_create) */
  HKV_ERR_NULL_POINTER = -3,  /* a required pointer is NULL */
  HKV_ERR_CAPACITY = -4,      /* an append would exceed max_blocks_per_seq or num_phys_blocks */
  HKV_ERR_WORKSPACE = -5,     /* workspace pointer NULL or smaller than hkv_workspace_bytes */
  HKV_ERR_HIP = -6,           /* a HIP runtime call or kernel launch failed */
  HKV_ERR_ALIGNMENT = -7,     /* a buffer is not aligned as documented */
  HKV_ERR_OUT_OF_MEMORY = -8  /* a host-side allocation of the library failed (nothing was launched) */
} hkv_status;

/* One cold block header, 16 bytes (Hybrid KV Cache page 3.2: each
 * block_header element is 16 bytes; V4 architecture page 2.2: a cold page
 * entry is a physical address plus a valid length).  The per-head scales do
 * not fit in 16 bytes, so they live in the `scales` array indexed by
 * phys_block.
 *   phys_block     caller-assigned physical block id in [0, num_phys_blocks)
 *                  for every logical block the sequence may reach; the
 *                  library never changes it.
 *   n_valid        tokens stored in the block (written by hkv_append).
 *   logical_block  index of the block in its sequence (written by hkv_append).
 *   flags          reserved, written as 0. */
typedef struct {
  int32_t phys_block;
  int32_t n_valid;
  int32_t logical_block;
  uint32_t flags;
} hkv_block_header;

/* Cache descriptor: pointers to caller-owned buffers, sized with
 * hkv_cache_sizes.  Layouts (H = n_kv_heads, d = head_dim, T = hot_tokens,
 * S = block_size, P = num_phys_blocks):
 *   hot      fp16 [batch][H][T][2][d]; ring slot = token position mod T;
 *            K then V of one token adjacent ("interleaved per token").
 *            Base 512-byte aligned (Hybrid KV Cache page 3.2).
 *   tail     fp16 [batch][H][2][S][d]; FP16 originals of each sequence's
 *            partially filled last cold block (row-major [token][channel]).
 *   cold     [P][H][2][tile bytes]; one tile per (physical block, kv-head,
 *            K|V) of S*d elements: 8-bit codes (8 KiB at S=64, d=128), 4-bit
 *            codes (4 KiB) or fp16 values (16 KiB, quant_bits 0).  A tile is
 *            made of 16-byte chunks of E elements (E = 16, 32 or 8).  K tiles:
 *            chunk (k, t) = channels E*k .. E*k+E-1 of token t, at byte
 *            (k*S + t)*16.  V tiles: chunk (v, c) = tokens E*v .. E*v+E-1 of
 *            channel c, at byte (v*d + c)*16.  Element e of a chunk is byte e
 *            (8-bit code + 128, so code -127..127 is stored 1..255 and code 0
 *            as 0x80), a half-byte (4-bit code + 8, so code -7..7 is stored
 *            1..15; each 32-bit word of a chunk holds elements 8j..8j+3 in
 *            the low half-bytes of its bytes 0..3 and 8j+4..8j+7 in the high
 *            ones) or the fp16 at bytes 2e, 2e+1.  Rows t >= n_valid hold
 *            code 0 (value 0).
 *   scales   fp32 [P][H][2]  (K scale, V scale).
 *   headers  hkv_block_header [batch][max_blocks_per_seq].
 *   seq_len_dev   int32 [batch] device: tokens cached per sequence.
 *   seq_len_host  int32 [batch] host mirror of seq_len_dev, used to plan
 *            launches and check capacity; hkv_append updates both.
 *   quant_err     optional (NULL = off) device fp32 [P][H][2]: debug statistic
 *            (Hybrid KV Cache page 6.3, kv_cache_debug: quantisation-error
 *            statistics).  Every append and fused step writes, for each
 *            (block, kv-head, K|V) tile it codes, the largest |x - code*scale|
 *            over the tile's valid elements, in fp32 (0 for fp16 tiles).
 *   entropy       optional (NULL = off) device fp32 [batch][n_q_heads]: debug
 *            statistic (KV Cache reuse page 6: monitor attention entropy).
 *            Every decode (dense, sparse, fused, no-alloc) writes the entropy
 *            -sum p ln p (nats) of each query head's softmax over the tokens it
 *            attends, computed as lse - E_p[z] from the same fp32 online
 *            softmax.
 *            A decode with entropy set runs a kernel variant that carries the
 *            statistic, under a static launch plan (no dynamic block claims,
 *            so long contexts decode more slowly); with entropy NULL the
 *            kernels hold no register for it.
 * A new cache is all zero except headers[].phys_block; every buffer except
 * hot must be 16-byte aligned.  The quantisation-error statistic costs a few
 * instructions per coded tile when enabled and nothing else. */
typedef struct {
  int32_t batch;
  int32_t max_blocks_per_seq;
  int32_t num_phys_blocks;
  void* hot;
  void* tail;
  int8_t* cold;
  float* scales;
  hkv_block_header* headers;
  int32_t* seq_len_dev;
  int32_t* seq_len_host;
  float* quant_err;  /* optional debug statistic, NULL = off */
  float* entropy;    /* optional debug statistic, NULL = off */
} hkv_cache_desc;

/* Bytes of every cache buffer, for one configuration (see hkv_cache_sizes). */
typedef struct {
  size_t hot;
  size_t tail;
  size_t cold;
  size_t scales;
  size_t headers;
  size_t seq_len;
  int32_t max_blocks_per_seq;
  int32_t num_phys_blocks;
} hkv_cache_sizes_t;

/* Create a handle for one layer's cache protocol (Hybrid KV Cache page 3.1:
 * the hybrid_v2 protocol has three required fields hot_tokens,
 * quantization_bits, block_size; 4.2 reads them with defaults 32 / 8 / 64).
 *   HKV_ERR_INVALID_VALUE: hot_tokens not in {16, 32, 64, 128} (5.1 assert),
 *     block_size <= 0 or block_size % 8 != 0 (3.1, 5.1), quant_bits not in
 *     {0, 4, 8} (3.1 allows 4 and 8; 5.2 uses 0 for an FP16 cold zone),
 *     n_kv_heads < 1 or head_dim < 1.
 *   HKV_ERR_UNSUPPORTED: protocol-valid values this library does not build:
 *     block_size != 64, head_dim not in {64, 128}.  All three widths are
 *     built: quant_bits 8 (INT8 codes), 4 (INT4 codes, two per byte) and 0
 *     (FP16 cold zone); see the cold-tile layouts above.
 *   HKV_ERR_NULL_POINTER: out is NULL.
 *   HKV_ERR_OUT_OF_MEMORY: the handle could not be allocated.
 * On success *out owns a small host object released by hkv_destroy. */
hkv_status hkv_create(int n_kv_heads, int head_dim, int hot_tokens, int block_size, int quant_bits,
                      hkv_handle* out);

/* Release a handle (NULL is accepted). Pending events of the timing state are
 * waited for.  Buffers are the caller's and are not touched. */
hkv_status hkv_destroy(hkv_handle h);

/* Buffer sizes for `batch` sequences of at most `max_tokens_per_seq` tokens
 * each and a pool of `num_phys_blocks` cold blocks (0 = batch *
 * max_blocks_per_seq, a dense pool).  max_blocks_per_seq =
 * ceil(max(0, max_tokens_per_seq - hot_tokens) / block_size).
 * HKV_ERR_INVALID_VALUE for negative counts or batch < 1. */
hkv_status hkv_cache_sizes(hkv_handle h, int batch, int64_t max_tokens_per_seq, int64_t num_phys_blocks,
                           hkv_cache_sizes_t* out);

/* The same sizes as hkv_cache_sizes, as a plain array of six byte counts in
 * the order hot, tail, cold, scales, headers, seq_len (the layouts above; a
 * dense pool when num_phys_blocks is 0).  HKV_ERR_INVALID_VALUE for negative
 * counts, batch < 1 or sizes past the int32 block-id range;
 * HKV_ERR_NULL_POINTER if h or bytes_out is NULL. */
hkv_status hkv_sizes(hkv_handle h, int batch, int max_tokens_per_seq, int num_phys_blocks, size_t bytes_out[6]);

/* Header-table size of one sequence (Hybrid KV Cache page 5.4: blocks =
 * ceil(tokens / block_size), about 16 bytes per block): *n_blocks =
 * ceil(max(0, total_tokens - hot_tokens) / block_size), *bytes = 16 *
 * *n_blocks.  Validates hot_tokens and block_size with the rules of
 * hkv_create but needs no handle, so protocol-valid block sizes that are not
 * built (e.g. 256) can be sized. */
hkv_status hkv_header_table_bytes(int hot_tokens, int block_size, int64_t total_tokens, int64_t* n_blocks,
                                  size_t* bytes);

/* Workspace bytes needed by hkv_decode_attn (dense and sparse),
 * hkv_append_decode and hkv_topk_select on this cache with n_q_heads query
 * heads and a top-K budget k_sel (0 if top-K is not used).  The bound holds
 * for every length up to the cache's capacity, so one allocation serves all
 * later calls.  The workspace must be zero-filled before its first use: its
 * first bytes hold per-(sequence, kv-head) and per-sequence arrival counters
 * and per-(sequence, kv-head) block-claim counters, which every call leaves at
 * zero again.  Calls that share a workspace must be ordered on one stream.
 * The counters' extent depends on the cache's batch and kv-head count, and
 * the partials follow them: a workspace that served a cache of another batch
 * or kv-head count must be zero-filled again before it serves this one.
 * HKV_ERR_INVALID_VALUE if n_q_heads is not a positive multiple of
 * n_kv_heads or k_sel is outside [0, 512]. */
hkv_status hkv_workspace_bytes(hkv_handle h, const hkv_cache_desc* c, int n_q_heads, int k_sel, size_t* bytes);

/* Append n_new_host[b] new tokens to every sequence b (0 allowed) and move
 * the tokens that leave the hot zone into cold blocks (Hybrid KV Cache page
 * 2.1: hot = the most recent hot_tokens tokens in full FP16, cold = older
 * tokens as INT8 with a block-wise scale; 4.2: quantise the non-hot part).
 *   k_new, v_new  device fp16 [batch][max_n_new][n_kv_heads][head_dim]; row
 *                 i < n_new_host[b] of sequence b is token seq_len[b] + i.
 *   n_new_host    host int32 [batch], each in [0, max_n_new].
 * The values are finite fp16 (a block's scale is its largest magnitude; a
 * NaN or infinity gives that block undefined codes).
 * Every cold block touched by the append is (re-)quantised from its FP16
 * values; headers get n_valid/logical_block; the hot ring, tail shadow,
 * seq_len_dev and seq_len_host are updated.  The result does not depend on
 * how a token stream is split into appends.
 *   HKV_ERR_CAPACITY: some sequence would need more than max_blocks_per_seq
 *     cold blocks.  HKV_ERR_INVALID_VALUE: max_n_new < 0, a count outside
 *     [0, max_n_new] or a negative seq_len_host entry.
 * Physical ids outside [0, num_phys_blocks) are skipped by the kernels, never
 * written through. */
hkv_status hkv_append(hkv_handle h, const hkv_cache_desc* c, const void* k_new, const void* v_new,
                      const int32_t* n_new_host, int max_n_new, hipStream_t stream);

/* Single-token decode attention for every sequence:
 *   out[b][hq] = softmax(q[b][hq] . K^T / sqrt(d)) . V
 * over the FP16 hot tokens and the dequantised cold tokens of kv-head
 * hq / (n_q_heads / n_kv_heads), with one softmax over both zones (the
 * Hybrid KV Cache page 4.2 computes the hot part with FlashAttention-2 and
 * dequantises cold blocks lazily; a joint softmax replaces its concatenation
 * of the two outputs).  Split-K partials are merged with a log-sum-exp
 * combine.  When the plan gives a split 16 or more cold blocks (long
 * sequences, or more (sequence, kv-head) pairs than the GPU holds at once),
 * the blocks of a (sequence, kv-head) are claimed by whichever wave is free,
 * so repeated calls agree to float rounding, not bit for bit; other launches
 * are bitwise reproducible.
 *   q        device fp16 [batch][n_q_heads][head_dim].
 *   sel_idx  NULL for dense decode, or device int32 [batch][n_kv_heads][k_sel]
 *            of selected cold-token indices (as written by
 *            hkv_topk_select; -1 entries and out-of-range entries are
 *            ignored, duplicates count twice): attention then covers the
 *            hot zone plus exactly these cold tokens (KV Cache reuse page 2:
 *            only the selected tokens are loaded).
 *   k_sel    entries per (sequence, kv-head) of sel_idx, 1..512 when sel_idx
 *            is given, ignored otherwise.
 *   out      device fp16 [batch][n_q_heads][head_dim] (round to nearest even).
 *   lse      NULL or device fp32 [batch][n_q_heads]: natural-log
 *            log-sum-exp of the scaled logits q.k/sqrt(d).
 *   workspace/ws_bytes  device scratch of at least hkv_workspace_bytes.
 * HKV_ERR_INVALID_VALUE: a sequence with seq_len_host == 0, n_q_heads not a
 * multiple of n_kv_heads, k_sel out of range.  HKV_ERR_UNSUPPORTED: a
 * GQA group size other than 1, 2, 4 or 8. */
hkv_status hkv_decode_attn(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads,
                           const int32_t* sel_idx, int k_sel, void* out, float* lse, void* workspace,
                           size_t ws_bytes, hipStream_t stream);

/* hkv_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Arguments, results and errors are
 * those of hkv_decode_attn (dense when sel_idx is NULL, sparse otherwise); the
 * call allocates nothing, on the host or the device.
 * Its scratch (arrival and claim counters, split partials) is one fixed
 * 32 MiB device array of the library, one copy per GPU, held until the
 * process ends.  The first call on a device takes the array's address on that
 * device and clears it with a kernel on `stream` (and waits for it unless the
 * stream is being captured); every call leaves the counters at zero again.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one
 * GPU (different streams without ordering, several host threads) race and
 * must be serialised by the caller.
 *   HKV_ERR_WORKSPACE: the call would need more scratch than the array holds:
 *     counters are kept in its first 4 MiB (about 16000 (sequence, kv-head)
 *     pairs) and the split partials in the other 28 MiB (the hkv_workspace_bytes
 *     of the same arguments, less the counters, must fit); use hkv_decode_attn
 *     with a workspace instead.
 *   HKV_ERR_HIP: the scratch set-up or the launch failed. */
hkv_status hkv_decode_attn_noalloc(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads,
                                   const int32_t* sel_idx, int k_sel, void* out, float* lse, hipStream_t stream);

/* One decode step in one launch: hkv_append of exactly one new token per
 * sequence followed by the dense hkv_decode_attn of q against the updated
 * cache (Hybrid KV Cache page 2.1 and 4.2: the token leaving the hot zone is
 * quantised into its cold block, then the query attends hot plus cold).  The
 * cache contents, out and lse are those of the two calls made in that order;
 * the append's work runs inside the decode launch instead of in a launch of
 * its own.
 *   k_new, v_new  device fp16 [batch][n_kv_heads][head_dim]: the new token
 *                 (position seq_len[b]) of every sequence.
 *   q, n_q_heads, out, lse, workspace, ws_bytes  as for hkv_decode_attn
 *                 (dense).
 * seq_len_dev and seq_len_host are incremented by one.  With at most 256
 * sequences the launch takes the lengths before the append from seq_len_host
 * (copied into its arguments) and only writes seq_len_dev; with more it reads
 * seq_len_dev.  Either way the two must hold the same lengths, as after every
 * call of this library.
 *   HKV_ERR_CAPACITY: a sequence would need more than max_blocks_per_seq
 *     cold blocks.  HKV_ERR_INVALID_VALUE: n_q_heads not a multiple of
 *     n_kv_heads or a negative seq_len_host entry.  HKV_ERR_UNSUPPORTED: a
 *     GQA group size other than 1, 2, 4 or 8, or block_size other than 64.
 *   HKV_ERR_ALIGNMENT: k_new, v_new, q or workspace not 16-byte aligned. */
hkv_status hkv_append_decode(hkv_handle h, const hkv_cache_desc* c, const void* k_new, const void* v_new,
                             const void* q, int n_q_heads, void* out, float* lse, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* HySparse-style top-K selection per (sequence, kv-head) over the cold
 * tokens (KV Cache reuse page 2 and 2.1):
 *   c_t = mean over the kv-head's query heads of cos(q_hq, k_t) in fp32
 *         (cos := 0 for a zero norm; the learned projection is taken as the
 *         identity; cosine is invariant to the block scale, so INT8 codes are
 *         scored directly),
 *   p_t = softmax of c inside each 64-token window (= cold block, valid
 *         tokens only),
 *   out_idx[b][h] = the k largest p (ties to the lower token index), in
 *         ascending token order, padded with -1 when fewer than k cold tokens
 *         exist (the page's fixed max_K = 512 with masked padding).
 *   k        1..512.  out_idx device int32 [batch][n_kv_heads][k].
 * HKV_ERR_UNSUPPORTED: block_size other than 64 (windows are cold blocks). */
hkv_status hkv_topk_select(hkv_handle h, const hkv_cache_desc* c, const void* q, int n_q_heads, int k,
                           int32_t* out_idx, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Compacted sparse store (KV Cache reuse page 2: the Index-Aware Cache
 * Layout re-packs the KV of the selected top-K tokens into a compact
 * "effective" block, and only that block is loaded; 2.1: blocks aligned to
 * 256 bytes and padded to a power of two).  A store holds, per (sequence,
 * kv-head), the valid entries of a selection in selection order (-1 and
 * out-of-range entries skipped, duplicates kept), in units of 64 tokens; a
 * unit is one K tile and one V tile in the cold-block chunk layouts (2 x tile
 * bytes: 16 KiB for 8-bit codes at head_dim 128), and every stored token keeps
 * its own block's K and V scales.  Layout (this library's): int32 counts
 * [batch][H]; at the next 256-byte boundary float2 scales
 * [batch][H][U][64]; at the next 256-byte boundary the units
 * [batch][H][U][2][tile bytes]; U = ceil(k_sel / 64).  The store is a copy:
 * it describes the cache as it was when hkv_sparse_compact ran (an append
 * that re-quantises a selected token's block is not reflected).
 *
 * Bytes of a store for `batch` sequences and selections of width k_sel.
 * HKV_ERR_INVALID_VALUE: batch < 1 or k_sel outside [1, 512]. */
hkv_status hkv_sparse_store_bytes(hkv_handle h, int batch, int k_sel, size_t* bytes);

/* Build a compacted store from a selection.
 *   sel_idx  device int32 [batch][n_kv_heads][k_sel] (as written by
 *            hkv_topk_select; the entry rules of hkv_decode_attn).
 *   store    device, 256-byte aligned, at least hkv_sparse_store_bytes.
 * HKV_ERR_WORKSPACE: store_bytes too small.  HKV_ERR_UNSUPPORTED: block_size
 * other than 64.  One launch of one workgroup per (unit, kv-head, sequence). */
hkv_status hkv_sparse_compact(hkv_handle h, const hkv_cache_desc* c, const int32_t* sel_idx, int k_sel, void* store,
                              size_t store_bytes, hipStream_t stream);

/* Decode over the hot zone plus the tokens of a compacted store (built by
 * hkv_sparse_compact for this cache, batch and k_sel): the result of the sparse
 * hkv_decode_attn with the selection the store was built from, reading only
 * the store's units and the hot zone.
 *   workspace  at least hkv_workspace_bytes(h, c, n_q_heads, k_sel).
 * Errors as hkv_decode_attn (sparse). */
hkv_status hkv_decode_attn_compact(hkv_handle h, const hkv_cache_desc* c, const void* store, int k_sel, const void* q,
                                   int n_q_heads, void* out, float* lse, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* hkv_status_string(hkv_status st);

/* Text describing the most recent HKV_ERR_HIP returned on the calling thread
 * (which HIP call failed and its hipError_t name); "" if none.  The pointer
 * stays valid until the next failing call on the same thread. */
const char* hkv_last_error_detail(void);

/* Kernel timing (profiling aid).  When enabled on a handle, every kernel the
 * handle launches is launched with a start/stop hipEvent pair recorded by the
 * dispatch itself (hipExtLaunchKernelGGL), so the measured interval is the
 * kernel's own execution on `stream`.  hkv_timing_read waits for the pending
 * events of one kernel kind and returns their summed milliseconds and count
 * (and clears them when reset != 0). */
typedef enum {
  HKV_KERNEL_APPEND = 0,        /* append/quantise (single-pass or first of two) */
  HKV_KERNEL_APPEND_RING = 1,   /* second pass of a multi-block append */
  HKV_KERNEL_DECODE = 2,        /* dense decode (splits + hot zone + combine, one launch) */
  HKV_KERNEL_DECODE_SPARSE = 3, /* sparse decode over selected tokens, one launch */
  HKV_KERNEL_TOPK_SCORE = 4,
  HKV_KERNEL_TOPK_SELECT = 5,
  HKV_KERNEL_APPEND_DECODE = 6, /* fused one-token append + dense decode, one launch */
  HKV_KERNEL_SPARSE_COMPACT = 7, /* building a compacted sparse store */
  HKV_KERNEL_DECODE_COMPACT = 8, /* decode over a compacted sparse store */
  HKV_KERNEL_KINDS = 9
} hkv_kernel_kind;

hkv_status hkv_timing_enable(hkv_handle h, int enable);

/* Phase timestamps (measurement aid, like the timing state).  While buf is
 * not NULL, every decode launch of the handle (hkv_decode_attn and its
 * no-allocation form, hkv_decode_attn_compact, hkv_append_decode) writes, per
 * workgroup, 8 uint64 readings of the GPU's constant 100 MHz clock
 * (s_memrealtime) to buf[w*8 + i], w = (sequence*H + kv_head)*nparts + part,
 * nparts = the launch's workgroups per (sequence, kv-head) (cold splits, then
 * the hot zone; for the fused step, in place of the hot zone's, the append
 * workgroup, which attends the new hot window and then appends):
 *   [0] workgroup start, [1] its partial records stored, [2] its arrival
 *   counted, [3] merge done (0 unless this workgroup merged);
 *   append workgroup of the fused step also: [4] its hot window attended
 *   (its first loads included), [5] its codes staged (0 without a valid
 *   block), [6] its code stores issued, [7] its block attended.  Other slots
 *   are not written.
 * Workgroups past bytes / 64 are not recorded; the caller clears buf.  NULL
 * turns it off.  The clock is the same on every die.
 * HKV_ERR_ALIGNMENT: buf not 8-byte aligned. */
hkv_status hkv_phase_stamps(hkv_handle h, uint64_t* buf, size_t bytes);

/* Launch-plan override (testing and tuning aid; like the timing state, it is
 * the handle's only other mutable state).  nsplit > 0 makes every dense decode
 * and fused step use a static plan of (at most) nsplit cold splits per
 * (sequence, kv-head), without block claims (results then agree bit for bit
 * between calls, and across split counts to fp32 rounding); claim_workgroups
 * > 0 sets the grid of plans that claim blocks.  0 restores the automatic
 * choice.  Workspace sizes queried after the call account for nsplit.
 * HKV_ERR_INVALID_VALUE: nsplit outside [0, 128] or claim_workgroups outside
 * [0, 65536]. */
hkv_status hkv_plan_override(hkv_handle h, int nsplit, int claim_workgroups);
hkv_status hkv_timing_read(hkv_handle h, int kind, double* total_ms, int64_t* count, int reset);

/* Streaming read probe (measurement aid, not part of the cache protocol): one
 * launch of `workgroups` x `threads` threads reads the `bytes` bytes at `src`
 * once with 16-byte non-temporal loads, the access pattern of the cold-tile
 * streams.  Its duration is the read floor that a one-launch decode over the
 * same number of bytes is measured against.
 *   src   device, 16-byte aligned; bytes a multiple of 16.
 *   sink  device uint32 [workgroups * threads]; written only if a lane's
 *         folded data equals a fixed sentinel (it keeps the loads alive).
 * HKV_ERR_INVALID_VALUE: threads not a multiple of 64 in [64, 1024],
 * workgroups < 1 or bytes % 16 != 0. */
hkv_status hkv_read_probe(const void* src, size_t bytes, int workgroups, int threads, uint32_t* sink,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HKV_H_ */
