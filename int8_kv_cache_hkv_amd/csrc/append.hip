// Append / spill / quantise kernels (gfx950).
//
// Hybrid KV Cache page, 2.1: the hot zone keeps the full FP16 KV of the most
// recent hot_tokens tokens; older tokens form the cold zone, stored as INT8
// with a block-wise scale.  4.2 (step 2): the non-hot part is quantised.
// Scale per (block, kv-head, K|V): s = fl32(max|x| / 127); code =
// clamp(rint(fl32(x / s)), -127, 127), round half to even.  A partially
// filled block always holds the codes of its current tokens, so every block
// an append touches is re-quantised from FP16 (older tokens of a partial block
// come from the per-sequence tail shadow).
//
// Two launches, in stream order (multi-block appends; the single-pass
// append_step_kernel below serves appends that touch at most two blocks):
//   append_quant_kernel  one workgroup per (sequence, touched block, kv-head):
//                        gathers the block's FP16 rows (tail shadow, hot ring,
//                        new tokens), reduces max|x|, divides and rounds, and
//                        writes the codes in the tile layouts the decode
//                        kernels stream, plus scales and the block header.
//   append_ring_kernel   one workgroup per sequence: copies the new partial
//                        block's FP16 rows into the tail shadow, then writes
//                        the new tokens into the hot ring (after every read of
//                        the slots they replace), then publishes seq_len.
#include <hip/hip_ext.h>

#include "hkv_device.h"

namespace hkv {

namespace detail {

template <int D>
__global__ __launch_bounds__(kThreads) void append_quant_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int TPT = kThreads / S;     // threads per token row
  constexpr int CPT = D / TPT;          // channels per thread (32 or 16)
  constexpr int LDS_ROW = D + 16;       // padded staging row (bytes), 16-byte aligned
  __shared__ __align__(16) int8_t stage[S * LDS_ROW];
  __shared__ float red[kWaves];

  const CacheView& c = p.c;
  const int H = c.H, T = c.T;
  const int wg = blockIdx.x;
  const int h = wg % H;
  const int rest = wg / H;
  const int jj = rest % p.touched_max;
  const int bl = rest / p.touched_max;
  if (bl >= p.n_seq) return;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  if (nn <= 0) return;
  const int n0 = c.seq_len[b];
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  if (cold1 <= cold0) return;
  const int j = cold0 / S + jj;
  if (j * S >= cold1 || j >= c.max_blocks) return;
  hkv_block_header* hdr = c.headers + static_cast<size_t>(b) * c.max_blocks + j;
  const int phys = hdr->phys_block;
  if (phys < 0 || phys >= c.num_phys) return;
  const int valid = min(S, cold1 - j * S);

  const int tid = threadIdx.x;
  const int t = tid / TPT;              // token row inside the block
  const int part = tid % TPT;           // channel slice
  const int pos = j * S + t;

  for (int kv = 0; kv < 2; ++kv) {
    // ---- gather the FP16 row slice of token t
    const _Float16* row = nullptr;
    if (t < valid) {
      if (pos < cold0) {
        row = c.tail + ((static_cast<size_t>(b) * H + h) * 2 + kv) * S * D + static_cast<size_t>(t) * D;
      } else if (pos < n0) {
        row = c.hot + (((static_cast<size_t>(b) * H + h) * T + (pos % T)) * 2 + kv) * D;
      } else {
        const _Float16* src = kv ? p.v_new : p.k_new;
        row = src + ((static_cast<size_t>(b) * p.max_n_new + (pos - n0)) * H + h) * D;
      }
    }
    float x[CPT];
    if (row) {
      const uint4* r4 = reinterpret_cast<const uint4*>(row + part * CPT);
#pragma unroll
      for (int v = 0; v < CPT / 8; ++v) {
        uint4 w = r4[v];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t u = word_of(w, i);
          x[v * 8 + 2 * i] = half_lo(u);
          x[v * 8 + 2 * i + 1] = half_hi(u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < CPT; ++i) x[i] = 0.f;
    }
    // ---- m = max |x| over the block (exact: every candidate is an fp16 value)
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) m = fmaxf(m, fabsf(x[i]));
    m = wave_max(m);
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w]);
    // ---- s = fl32(m / 127): IEEE fp32 division (correctly rounded)
    const float s = m / 127.0f;
    // ---- codes = clamp(rint(fl32(x / s)), -127, 127), round half to even
    int8_t* srow = stage + t * LDS_ROW + part * CPT;
#pragma unroll
    for (int i = 0; i < CPT; i += 4) {
      uint32_t packed = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float qv = 0.f;
        if (s > 0.f) qv = fminf(127.f, fmaxf(-127.f, __builtin_rintf(x[i + k] / s)));
        packed |= (static_cast<uint32_t>(static_cast<int>(qv)) & 0xffu) << (8 * k);
      }
      *reinterpret_cast<uint32_t*>(srow + i) = packed;
    }
    __syncthreads();
    // ---- write the tile in its streaming layout (16-byte vectors, coalesced)
    int8_t* tile = c.cold + tile_offset(phys, h, kv, H, S, D);
    constexpr int NVEC = S * D / 16;
    for (int vi = tid; vi < NVEC; vi += kThreads) {
      uint4 out;
      if (kv == 0) {
        // K: vector (channel chunk dc, token tt) holds channels dc*16..dc*16+15 of token tt
        const int dc = vi / S, tt = vi % S;
        out = *reinterpret_cast<const uint4*>(stage + tt * LDS_ROW + dc * 16);
      } else {
        // V: vector (token chunk tc, channel cc) holds tokens tc*16..tc*16+15 of channel cc
        const int tc = vi / D, cc = vi % D;
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t acc = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            acc |= static_cast<uint32_t>(static_cast<uint8_t>(stage[(tc * 16 + i * 4 + k) * LDS_ROW + cc])) << (8 * k);
          wv[i] = acc;
        }
        out = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      reinterpret_cast<uint4*>(tile)[vi] = out;
    }
    if (tid == 0) c.scales[(static_cast<size_t>(phys) * H + h) * 2 + kv] = s;
    __syncthreads();  // stage and red are reused by the V pass
  }
  if (h == 0 && tid == 0) {
    hdr->n_valid = valid;
    hdr->logical_block = j;
    hdr->flags = 0u;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void append_ring_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int VPR = D / 8;            // 16-byte vectors per (token, head, K|V) row
  const CacheView& c = p.c;
  const int H = c.H, T = c.T;
  const int bl = blockIdx.x;
  if (bl >= p.n_seq) return;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  if (nn <= 0) return;
  const int n0 = c.seq_len[b];
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  const int tid = threadIdx.x;

  // (1) FP16 shadow of the new partial last block (rows already there stay)
  const int jf = cold1 / S;
  if ((cold1 % S) != 0 && jf < c.max_blocks) {
    const int lo = max(jf * S, cold0), hi = cold1;
    const int items = (hi - lo) * H * 2 * VPR;
    for (int it = tid; it < items; it += kThreads) {
      const int v = it % VPR;
      int r = it / VPR;
      const int kv = r % 2;
      r /= 2;
      const int h = r % H;
      const int pos = lo + r / H;
      const _Float16* src;
      if (pos < n0) {
        src = c.hot + (((static_cast<size_t>(b) * H + h) * T + (pos % T)) * 2 + kv) * D;
      } else {
        src = (kv ? p.v_new : p.k_new) + ((static_cast<size_t>(b) * p.max_n_new + (pos - n0)) * H + h) * D;
      }
      _Float16* dst = c.tail + ((static_cast<size_t>(b) * H + h) * 2 + kv) * S * D + static_cast<size_t>(pos - jf * S) * D;
      reinterpret_cast<uint4*>(dst)[v] = reinterpret_cast<const uint4*>(src)[v];
    }
  }
  __syncthreads();  // ring slots read above are overwritten below
  // (2) new tokens that remain hot go to ring slot pos mod T
  {
    const int lo = max(n0, n1 - T), hi = n1;
    const int items = (hi - lo) * H * 2 * VPR;
    for (int it = tid; it < items; it += kThreads) {
      const int v = it % VPR;
      int r = it / VPR;
      const int kv = r % 2;
      r /= 2;
      const int h = r % H;
      const int pos = lo + r / H;
      const _Float16* src = (kv ? p.v_new : p.k_new) + ((static_cast<size_t>(b) * p.max_n_new + (pos - n0)) * H + h) * D;
      _Float16* dst = c.hot + (((static_cast<size_t>(b) * H + h) * T + (pos % T)) * 2 + kv) * D;
      reinterpret_cast<uint4*>(dst)[v] = reinterpret_cast<const uint4*>(src)[v];
    }
  }
  __syncthreads();
  if (tid == 0) c.seq_len[b] = n1;
}

// Single-pass append, one workgroup per (sequence, kv-head), for appends that
// touch at most a couple of cold blocks per sequence (a decode step touches
// one).  Everything one kv-head of one sequence owns (its touched tiles, tail
// shadow rows and hot-ring slots) is handled by one workgroup in program
// order, so no second launch is needed; the cached length comes from the host
// mirror (kernel argument), so no workgroup reads seq_len while another
// publishes it.
//
// Block scale reuse: s = fl32(m / 127) is monotonic and injective on fp16
// maxima, so when fl32(m_new / 127) <= s_old for the rows being added, the
// block maximum and scale are unchanged and the old rows keep their codes;
// only the new rows are coded.  Otherwise the whole block is re-quantised
// from its FP16 rows.  Both paths give the codes a full re-quantisation gives.
template <int D>
__global__ __launch_bounds__(kThreads) void append_step_kernel(AppendParams p) {
  constexpr int S = kBlockSize;
  constexpr int TPT = kThreads / S;     // threads per token row
  constexpr int CPT = D / TPT;          // channels per thread
  constexpr int LDS_ROW = D + 16;
  constexpr int VPR = D / 8;            // 16-byte vectors per fp16 row
  __shared__ __align__(16) int8_t stage[S * LDS_ROW];
  __shared__ float red[kWaves], red2[kWaves];

  const CacheView& c = p.c;
  const int H = c.H, T = c.T;
  const int h = blockIdx.x % H;
  const int bl = blockIdx.x / H;
  if (bl >= p.n_seq) return;
  const int b = p.b0 + bl;
  const int nn = p.n_new[bl];
  if (nn <= 0) return;
  const int n0 = p.n0[bl];
  const int n1 = n0 + nn;
  const int cold0 = n0 > T ? n0 - T : 0;
  const int cold1 = n1 > T ? n1 - T : 0;
  const int tid = threadIdx.x;
  const int t = tid / TPT, part = tid % TPT;
  const size_t bh = static_cast<size_t>(b) * H + h;

  auto row_ptr = [&](int pos, int kv) -> const _Float16* {
    if (pos < n0) return c.hot + ((bh * T + (pos % T)) * 2 + kv) * D;
    return (kv ? p.v_new : p.k_new) + ((static_cast<size_t>(b) * p.max_n_new + (pos - n0)) * H + h) * D;
  };
  auto block_max2 = [&](float& m0, float& m1) {
    m0 = wave_max(m0);
    m1 = wave_max(m1);
    if ((tid & 63) == 0) {
      red[tid >> 6] = m0;
      red2[tid >> 6] = m1;
    }
    __syncthreads();
    float r0 = red[0], r1 = red2[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      r0 = fmaxf(r0, red[w]);
      r1 = fmaxf(r1, red2[w]);
    }
    __syncthreads();
    m0 = r0;
    m1 = r1;
  };
  auto load_row = [&](const _Float16* row, float (&x)[CPT]) {
    const uint4* r4 = reinterpret_cast<const uint4*>(row + part * CPT);
#pragma unroll
    for (int v = 0; v < CPT / 8; ++v) {
      const uint4 wv = r4[v];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[v * 8 + 2 * i] = half_lo(word_of(wv, i));
        x[v * 8 + 2 * i + 1] = half_hi(word_of(wv, i));
      }
    }
  };

  for (int j = cold0 / S; j * S < cold1; ++j) {
    if (j >= c.max_blocks) break;
    const int v_old = j * S < cold0 ? cold0 - j * S : 0;   // rows already coded, FP16 in the tail shadow
    const int v_new = min(S, cold1 - j * S);
    const bool is_new = t >= v_old && t < v_new;
    // the new K and V rows do not depend on the block's physical id: load them together with the header
    float x[2][CPT];
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      if (is_new) {
        load_row(row_ptr(j * S + t, kv), x[kv]);
      } else {
#pragma unroll
        for (int i = 0; i < CPT; ++i) x[kv][i] = 0.f;
      }
    }
    hkv_block_header* hdr = c.headers + static_cast<size_t>(b) * c.max_blocks + j;
    const int phys = hdr->phys_block;
    float mnew[2] = {0.f, 0.f};
#pragma unroll
    for (int kv = 0; kv < 2; ++kv)
#pragma unroll
      for (int i = 0; i < CPT; ++i) mnew[kv] = fmaxf(mnew[kv], fabsf(x[kv][i]));
    block_max2(mnew[0], mnew[1]);
    if (phys < 0 || phys >= c.num_phys) continue;
    float* sp = c.scales + (static_cast<size_t>(phys) * H + h) * 2;
    const float s_old[2] = {v_old > 0 ? sp[0] : 0.f, v_old > 0 ? sp[1] : 0.f};
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {  // unrolled: x[kv] must stay in registers
      int8_t* tile = c.cold + tile_offset(phys, h, kv, H, S, D);
      if (v_old > 0 && mnew[kv] / 127.0f <= s_old[kv]) {
        // ---- scale unchanged: code only the new rows, in place
        const float so = s_old[kv];
        if (is_new) {
          int8_t q8[CPT];
#pragma unroll
          for (int i = 0; i < CPT; ++i)
            q8[i] = so > 0.f ? static_cast<int8_t>(fminf(127.f, fmaxf(-127.f, __builtin_rintf(x[kv][i] / so)))) : 0;
          if (kv == 0) {
#pragma unroll
            for (int ch = 0; ch < CPT / 16; ++ch) {
              const int dc = (part * CPT) / 16 + ch;
              uint32_t wv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                wv[i] = (static_cast<uint32_t>(static_cast<uint8_t>(q8[ch * 16 + 4 * i])) |
                         (static_cast<uint32_t>(static_cast<uint8_t>(q8[ch * 16 + 4 * i + 1])) << 8) |
                         (static_cast<uint32_t>(static_cast<uint8_t>(q8[ch * 16 + 4 * i + 2])) << 16) |
                         (static_cast<uint32_t>(static_cast<uint8_t>(q8[ch * 16 + 4 * i + 3])) << 24));
              reinterpret_cast<uint4*>(tile)[dc * S + t] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
          } else {
#pragma unroll
            for (int i = 0; i < CPT; ++i) tile[((t / 16) * D + part * CPT + i) * 16 + (t % 16)] = q8[i];
          }
        }
        continue;
      }
      // ---- (re-)quantise the whole block: old rows come back from the tail shadow
      float mblk = mnew[kv];
      if (v_old > 0) {
        if (t < v_old) load_row(c.tail + ((bh * 2 + kv) * S + t) * D, x[kv]);
        float mo = 0.f, dummy = 0.f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) mo = fmaxf(mo, fabsf(x[kv][i]));
        block_max2(mo, dummy);
        mblk = fmaxf(mblk, mo);
      }
      const float s = mblk / 127.0f;
      int8_t* srow = stage + t * LDS_ROW + part * CPT;
#pragma unroll
      for (int i = 0; i < CPT; i += 4) {
        uint32_t packed = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float qv = 0.f;
          if (s > 0.f) qv = fminf(127.f, fmaxf(-127.f, __builtin_rintf(x[kv][i + k] / s)));
          packed |= (static_cast<uint32_t>(static_cast<int>(qv)) & 0xffu) << (8 * k);
        }
        *reinterpret_cast<uint32_t*>(srow + i) = packed;
      }
      __syncthreads();
      constexpr int NVEC = S * D / 16;
      for (int vi = tid; vi < NVEC; vi += kThreads) {
        uint4 out;
        if (kv == 0) {
          const int dc = vi / S, tt = vi % S;
          out = *reinterpret_cast<const uint4*>(stage + tt * LDS_ROW + dc * 16);
        } else {
          const int tc = vi / D, cc = vi % D;
          uint32_t wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t acc = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              acc |= static_cast<uint32_t>(static_cast<uint8_t>(stage[(tc * 16 + i * 4 + k) * LDS_ROW + cc])) << (8 * k);
            wv[i] = acc;
          }
          out = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        reinterpret_cast<uint4*>(tile)[vi] = out;
      }
      if (tid == 0) sp[kv] = s;
      __syncthreads();
    }
    if (h == 0 && tid == 0) {
      hdr->n_valid = v_new;
      hdr->logical_block = j;
      hdr->flags = 0u;
    }
  }
  __syncthreads();  // every read of the tail shadow and of spilled ring slots is done
  // FP16 shadow of the new partial last block (rows already there stay)
  const int jf = cold1 / S;
  if ((cold1 % S) != 0) {
    const int lo = max(jf * S, cold0), hi = cold1;
    for (int it = tid; it < (hi - lo) * 2 * VPR; it += kThreads) {
      const int v = it % VPR;
      const int kv = (it / VPR) % 2;
      const int pos = lo + it / (2 * VPR);
      reinterpret_cast<uint4*>(c.tail + ((bh * 2 + kv) * S + (pos - jf * S)) * D)[v] =
          reinterpret_cast<const uint4*>(row_ptr(pos, kv))[v];
    }
  }
  __syncthreads();  // ring slots read above are overwritten below
  {
    const int lo = max(n0, n1 - T), hi = n1;
    for (int it = tid; it < (hi - lo) * 2 * VPR; it += kThreads) {
      const int v = it % VPR;
      const int kv = (it / VPR) % 2;
      const int pos = lo + it / (2 * VPR);
      reinterpret_cast<uint4*>(c.hot + ((bh * T + (pos % T)) * 2 + kv) * D)[v] =
          reinterpret_cast<const uint4*>(row_ptr(pos, kv))[v];
    }
  }
  if (h == 0 && tid == 0) c.seq_len[b] = n1;
}

template <typename K>
hipError_t launch1(K kernel, int grid, const AppendParams& p, const LaunchCtx& ctx) {
  if (grid <= 0) return hipSuccess;
  if (ctx.start) {
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, ctx.stream, ctx.start, ctx.stop, 0, p);
  } else {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), 0, ctx.stream, p);
  }
  return hipGetLastError();
}

}  // namespace detail

using namespace detail;

hipError_t launch_append(const AppendParams& p, const LaunchCtx& quant_ctx, const LaunchCtx& ring_ctx) {
  if (p.single_pass) {
    return p.c.D == 128 ? launch1(append_step_kernel<128>, p.n_seq * p.c.H, p, quant_ctx)
                        : launch1(append_step_kernel<64>, p.n_seq * p.c.H, p, quant_ctx);
  }
  const int qgrid = p.touched_max > 0 ? p.n_seq * p.touched_max * p.c.H : 0;
  hipError_t e;
  if (p.c.D == 128) {
    e = launch1(append_quant_kernel<128>, qgrid, p, quant_ctx);
    if (e == hipSuccess) e = launch1(append_ring_kernel<128>, p.n_seq, p, ring_ctx);
  } else {
    e = launch1(append_quant_kernel<64>, qgrid, p, quant_ctx);
    if (e == hipSuccess) e = launch1(append_ring_kernel<64>, p.n_seq, p, ring_ctx);
  }
  return e;
}

}  // namespace hkv
