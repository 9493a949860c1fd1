"""Plain, slow fp64 CPU oracle for hybrid FP16-hot / INT8-cold KV-cache decode.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do. It shares no code with the HIP library: every step is
written here from the pages' definitions, in NumPy, in float64 unless a step
fixes a narrower type.

Sources (three web pages; cited by short title and section):

* "Hybrid KV Cache page" -- "DeepSeek V4 hybrid KV Cache inference
  optimisation: hands-on analysis" (tqpw.cn news 44343).
* "KV Cache reuse page" -- "KV Cache reuse: the key to LLM-inference memory
  and throughput" (yfxerp.com news 372023), HySparse part.
* "V4 architecture page" -- "DeepSeek V4 architecture: MoE dynamic loading and
  hierarchical KV cache" (xxmr.cn news 3419).

What is computed (readings where the pages are silent are marked READING):

1. History split. The hot zone is the full-precision KV of the most recent
   ``hot_tokens`` tokens, never quantised (Hybrid KV Cache page, 2.1 and
   3.1). Everything older is the cold zone, cut into ``block_size``-token
   blocks from token 0; the last block may be partial (READING: its codes are
   always those of its current valid tokens).
2. Block scale. One scale per (cold block, kv-head, K or V) ("INT8 with a
   block-wise scale", Hybrid KV Cache page 2.1; per-head granularity is a
   READING).  m = max |x| over the block's valid tokens and all channels;
   s = fl32(m / 127).  m is exact (fp16 -> fp64); the fp64 quotient rounded
   once to fp32 equals the correctly rounded fp32 quotient because
   53 >= 2*24 + 2 (double rounding is innocuous, Figueroa 1995).
3. Codes. q = clip(rint(fl32(x / s)), -127, 127), rint = round half to even;
   s == 0 gives all-zero codes (READING: symmetric absmax code, -128 unused).
4. Dequantisation x_hat = q * s, exact in fp64 (8-bit times 24-bit < 53 bits).
5. Decode. For query head hq of kv-head hq // G (contiguous GQA groups,
   READING), softmax(q . K^T / sqrt(d)) . V over every cached token, hot
   (fp16 values) and cold (dequantised), with one joint softmax (the printed
   patch concatenates two separate outputs, which is not attention; READING).
   Also lse = max z + ln sum exp(z - max z).
6. Top-K selection (KV Cache reuse page, 2 and 2.1). For each cold token t
   and kv-head, c_t = mean over the G query heads of cos(q_hq, k_hat_t)
   (READING for the GQA mean; the page has one query), cos := 0 when a norm
   is 0; the learned 128-dim projection is taken as the identity. Softmax
   inside each 64-token window (windows = cold blocks, valid tokens only),
   then the K largest window-probabilities, ties to the lower token index,
   returned ascending and padded with -1 to K (the page fixes max_K = 512
   with masked padding).
7. Sparse decode: step 5 restricted to the hot zone plus the selected cold
   tokens.
8. Header table sizing (Hybrid KV Cache page 5.4): one 16-byte header per
   cold block, blocks = ceil(cold tokens / block_size).
9. Cold-zone width (Hybrid KV Cache page 3.1: quantization_bits is 4 or 8,
   INT4 for L2 cold blocks; 5.2: quantization_bits 0 turns quantisation off
   and the cold zone stays FP16).  A b-bit code is the same symmetric absmax
   code with the largest magnitude L = 2^(b-1) - 1 (127 for INT8, 7 for INT4):
   s = fl32(m / L), q = clip(rint(fl32(x / s)), -L, L) (READING: the pages
   define neither code).  With 0 bits the cold tokens keep their fp16 values
   and the state records a scale of 1 for every (block, kv-head, K|V).
10. Debug statistics (Hybrid KV Cache page 6.3: a kv_cache_debug switch logs
   quantisation-error statistics every step; KV Cache reuse page 6: monitor
   the attention entropy, whose sudden drop signals lost context).  READING:
   the quantisation error of a (block, kv-head, K|V) tile is the largest
   |x - x_hat| over its valid elements (0 for an FP16 cold zone), and the
   entropy of a decode is -sum_t p_t ln p_t of each query head's attention
   distribution over the tokens it attends.
11. Compacted sparse store (KV Cache reuse page 2: the Index-Aware Cache
   Layout re-packs the KV of the selected top-K tokens into a compact block
   that is the only thing loaded; 2.1: aligned, padded blocks).  The store of
   a (sequence, kv-head) is its selected cold rows in selection order (masked
   and out-of-range entries skipped, duplicates kept), each with its own
   block's K and V scales; decoding over the hot zone plus the store is the
   sparse decode of item 7.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

HEADER_BYTES = 16  # Hybrid KV Cache page 3.2: each block_header element is 16 bytes


# --------------------------------------------------------------------------- quantisation
QUANT_BITS = (8, 4, 0)   # Hybrid KV Cache page 3.1 (4 or 8) and 5.2 (0 = FP16 cold zone)


def code_limit(bits: int = 8) -> int:
    """Largest code magnitude of the symmetric b-bit code: 2^(b-1) - 1 (127 at 8 bits, 7 at 4)."""
    if bits not in (8, 4):
        raise ValueError("only 8- and 4-bit cold blocks are quantised")
    return (1 << (bits - 1)) - 1


def block_scale(x_valid: np.ndarray, bits: int = 8) -> np.float32:
    """s = fl32(max|x| / L) over every element of one (block, kv-head, K|V) tile, L = code_limit(bits).

    Hybrid KV Cache page 2.1 (INT8 with a block-wise scale) and 3.1 (4 or 8
    bits); the formula is the symmetric absmax reading.
    """
    lim = code_limit(bits)
    x = np.asarray(x_valid)
    if x.size == 0:
        return np.float32(0.0)
    xd = x.astype(np.float64)
    if not np.all(np.isfinite(xd)):
        raise ValueError("cache inputs must be finite")
    m = float(np.max(np.abs(xd)))
    return np.float32(m / float(lim))


def quantize_codes(x_valid: np.ndarray, s: np.float32, bits: int = 8) -> np.ndarray:
    """Codes clip(rint(fl32(x / s)), -L, L) as int8 values (L = code_limit(bits)); zeros when s == 0."""
    lim = code_limit(bits)
    x = np.asarray(x_valid)
    if float(s) == 0.0:
        return np.zeros(x.shape, dtype=np.int8)
    quot = (x.astype(np.float64) / np.float64(s)).astype(np.float32)  # correctly rounded fp32 quotient
    q = np.rint(quot.astype(np.float64))                               # round half to even
    return np.clip(q, -lim, lim).astype(np.int8)


def dequantize(codes: np.ndarray, s: np.float32) -> np.ndarray:
    """x_hat = code * s in fp64 (exact; an FP16 cold zone stores its values with s = 1)."""
    return codes.astype(np.float64) * np.float64(s)


# --------------------------------------------------------------------------- cache state
@dataclasses.dataclass
class SequenceState:
    """Hybrid cache contents of one sequence as a pure function of its token history."""
    hot_tokens: int
    block_size: int
    n_tokens: int
    hot_k: np.ndarray        # fp16 [n_hot, H, d], position order
    hot_v: np.ndarray
    codes: np.ndarray        # [n_blk, H, 2, S, d]: int8 codes (8 or 4 bits) or fp16 values (0 bits);
                             # rows >= n_valid are 0
    scales: np.ndarray       # fp32 [n_blk, H, 2] (all 1 for an FP16 cold zone)
    n_valid: np.ndarray      # int64 [n_blk]
    quant_bits: int = 8

    @property
    def n_hot(self) -> int:
        return self.hot_k.shape[0]

    @property
    def n_cold(self) -> int:
        return self.n_tokens - self.n_hot

    @property
    def n_blocks(self) -> int:
        return self.codes.shape[0]


def split_history(n: int, hot_tokens: int) -> Tuple[int, int]:
    """(n_hot, n_cold): the most recent min(n, hot_tokens) tokens are hot (Hybrid KV Cache page 2.1)."""
    n_hot = min(n, hot_tokens)
    return n_hot, n - n_hot


def quantize_block(k_rows: np.ndarray, v_rows: np.ndarray, block_size: int, bits: int = 8
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Codes [H, 2, S, d] and scales [H, 2] of one cold block from its valid fp16 rows [n_valid, H, d].

    bits 0 (FP16 cold zone, Hybrid KV Cache page 5.2): the rows themselves, scale 1."""
    n_valid, n_heads, d = k_rows.shape
    if bits == 0:
        codes = np.zeros((n_heads, 2, block_size, d), dtype=np.float16)
        for c, rows in enumerate((k_rows, v_rows)):
            codes[:, c, :n_valid, :] = np.asarray(rows, dtype=np.float16).transpose(1, 0, 2)
        return codes, np.ones((n_heads, 2), dtype=np.float32)
    codes = np.zeros((n_heads, 2, block_size, d), dtype=np.int8)
    scales = np.zeros((n_heads, 2), dtype=np.float32)
    for h in range(n_heads):
        for c, rows in enumerate((k_rows, v_rows)):
            tile = rows[:, h, :]
            s = block_scale(tile, bits)
            scales[h, c] = s
            codes[h, c, :n_valid, :] = quantize_codes(tile, s, bits)
    return codes, scales


def build_state(k_hist: np.ndarray, v_hist: np.ndarray, hot_tokens: int, block_size: int,
                quant_bits: int = 8) -> SequenceState:
    """State after a sequence's whole history k_hist/v_hist (fp16 [n, H, d]) has been cached."""
    if quant_bits not in QUANT_BITS:
        raise ValueError("quantization_bits must be 8, 4 or 0")
    k_hist = np.asarray(k_hist, dtype=np.float16)
    v_hist = np.asarray(v_hist, dtype=np.float16)
    n, n_heads, d = k_hist.shape
    n_hot, n_cold = split_history(n, hot_tokens)
    n_blk = -(-n_cold // block_size)
    codes = np.zeros((n_blk, n_heads, 2, block_size, d), dtype=np.float16 if quant_bits == 0 else np.int8)
    scales = np.zeros((n_blk, n_heads, 2), dtype=np.float32)
    n_valid = np.zeros(n_blk, dtype=np.int64)
    for j in range(n_blk):
        lo, hi = j * block_size, min((j + 1) * block_size, n_cold)
        n_valid[j] = hi - lo
        codes[j], scales[j] = quantize_block(k_hist[lo:hi], v_hist[lo:hi], block_size, quant_bits)
    return SequenceState(hot_tokens, block_size, n, k_hist[n_cold:].copy(), v_hist[n_cold:].copy(),
                         codes, scales, n_valid, quant_bits)


def cold_kv(state: SequenceState, h: int) -> Tuple[np.ndarray, np.ndarray]:
    """Dequantised cold keys and values of kv-head h, fp64 [n_cold, d], token order."""
    ks, vs = [], []
    for j in range(state.n_blocks):
        nv = int(state.n_valid[j])
        ks.append(dequantize(state.codes[j, h, 0, :nv], state.scales[j, h, 0]))
        vs.append(dequantize(state.codes[j, h, 1, :nv], state.scales[j, h, 1]))
    d = state.hot_k.shape[2]
    if not ks:
        return np.zeros((0, d)), np.zeros((0, d))
    return np.concatenate(ks), np.concatenate(vs)


# --------------------------------------------------------------------------- attention
def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> Tuple[np.ndarray, float]:
    """softmax(q . K^T / sqrt(d)) . V for one query row, plus its log-sum-exp (fp64)."""
    d = q.shape[0]
    z = keys @ q / math.sqrt(d)
    zmax = float(np.max(z))
    e = np.exp(z - zmax)
    den = float(np.sum(e))
    return (e @ vals) / den, zmax + math.log(den)


def _group(n_q_heads: int, n_kv_heads: int) -> int:
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of kv-heads")
    return n_q_heads // n_kv_heads


def decode(q: np.ndarray, state: SequenceState, heads: Optional[Sequence[int]] = None
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention of one sequence: q fp16 [Hq, d] -> (out fp64 [Hq, d], lse fp64 [Hq])."""
    return _decode_over(q, state, None, heads)


def _decode_over(q: np.ndarray, state: SequenceState, sel: Optional[np.ndarray],
                 heads: Optional[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    n_q, d = q64.shape
    n_kv = state.hot_k.shape[1]
    g = _group(n_q, n_kv)
    if state.n_tokens == 0:
        raise ValueError("decode needs at least one cached token")
    out = np.full((n_q, d), np.nan)
    lse = np.full(n_q, np.nan)
    cache = {}
    for hq in (range(n_q) if heads is None else heads):
        h = hq // g
        if h not in cache:
            ck, cv = cold_kv(state, h)
            if sel is not None:
                keep = sel[h][sel[h] >= 0]
                ck, cv = ck[keep], cv[keep]
            keys = np.concatenate([ck, state.hot_k[:, h, :].astype(np.float64)])
            vals = np.concatenate([cv, state.hot_v[:, h, :].astype(np.float64)])
            cache = {h: (keys, vals)}
        keys, vals = cache[h]
        out[hq], lse[hq] = attend(q64[hq], keys, vals)
    return out, lse


# --------------------------------------------------------------------------- top-K (HySparse-style)
def token_scores(q: np.ndarray, state: SequenceState) -> np.ndarray:
    """c [H, n_cold]: per kv-head, mean over its query heads of cos(q_hq, k_hat_t)."""
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    n_q = q64.shape[0]
    n_kv = state.hot_k.shape[1]
    g = _group(n_q, n_kv)
    c = np.zeros((n_kv, state.n_cold))
    for h in range(n_kv):
        ck, _ = cold_kv(state, h)
        knorm = np.linalg.norm(ck, axis=1)
        acc = np.zeros(state.n_cold)
        for hq in range(h * g, (h + 1) * g):
            qn = float(np.linalg.norm(q64[hq]))
            dots = ck @ q64[hq]
            den = qn * knorm
            acc += np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
        c[h] = acc / g
    return c


def window_softmax(c: np.ndarray, n_valid: np.ndarray, block_size: int) -> np.ndarray:
    """Softmax of the scores inside each window (= cold block, valid tokens only), temperature 1."""
    p = np.zeros_like(c)
    for j, nv in enumerate(n_valid):
        lo, hi = j * block_size, j * block_size + int(nv)
        w = c[..., lo:hi]
        e = np.exp(w - np.max(w, axis=-1, keepdims=True))
        p[..., lo:hi] = e / np.sum(e, axis=-1, keepdims=True)
    return p


def topk_select(q: np.ndarray, state: SequenceState, k: int
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(idx int64 [H, k] ascending, -1-padded; p [H, n_cold]; tau [H] = k-th largest p, or -inf)."""
    p = window_softmax(token_scores(q, state), state.n_valid, state.block_size)
    n_kv = p.shape[0]
    idx = np.full((n_kv, k), -1, dtype=np.int64)
    tau = np.full(n_kv, -np.inf)
    for h in range(n_kv):
        order = sorted(range(state.n_cold), key=lambda t: (-p[h, t], t))  # larger p first, ties -> lower index
        chosen = sorted(order[:k])
        idx[h, :len(chosen)] = chosen
        if state.n_cold >= k:
            tau[h] = p[h, order[k - 1]]
    return idx, p, tau


def sparse_decode(q: np.ndarray, state: SequenceState, idx: np.ndarray,
                  heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over the hot zone plus the selected cold tokens idx [H, k] (-1 entries ignored)."""
    return _decode_over(q, state, np.asarray(idx), heads)


# --------------------------------------------------------------------------- compacted sparse store
@dataclasses.dataclass
class SparseStore:
    """Selected cold rows of one sequence per kv-head, in selection order (KV Cache reuse page 2)."""
    k_codes: list            # per kv-head: [m_h, d] codes (int8) or fp16 values
    v_codes: list
    k_scales: list           # per kv-head: [m_h] fp32 (the token's block scale)
    v_scales: list
    counts: np.ndarray       # int64 [H]: m_h, the valid entries of the selection


def sparse_store(state: SequenceState, idx: np.ndarray) -> SparseStore:
    """The compacted store of a selection idx [H, k]: for every entry 0 <= t < n_cold, the codes of
    cold token t (block t // S, row t % S) and its block's scales; other entries are skipped."""
    S = state.block_size
    d = state.hot_k.shape[2]
    ks, vs, kss, vss, cnt = [], [], [], [], []
    for h in range(idx.shape[0]):
        rows = [int(t) for t in idx[h] if 0 <= int(t) < state.n_cold]
        ks.append(np.array([state.codes[t // S, h, 0, t % S] for t in rows], dtype=state.codes.dtype).reshape(len(rows), d))
        vs.append(np.array([state.codes[t // S, h, 1, t % S] for t in rows], dtype=state.codes.dtype).reshape(len(rows), d))
        kss.append(np.array([state.scales[t // S, h, 0] for t in rows], dtype=np.float32))
        vss.append(np.array([state.scales[t // S, h, 1] for t in rows], dtype=np.float32))
        cnt.append(len(rows))
    return SparseStore(ks, vs, kss, vss, np.array(cnt, dtype=np.int64))


def decode_over_store(q: np.ndarray, state: SequenceState, store: SparseStore,
                      heads: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over the hot zone plus the rows of a compacted store (dequantised with their own scales)."""
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    n_q, d = q64.shape
    g = _group(n_q, state.hot_k.shape[1])
    out = np.full((n_q, d), np.nan)
    lse = np.full(n_q, np.nan)
    for hq in (range(n_q) if heads is None else heads):
        h = hq // g
        ck = store.k_codes[h].astype(np.float64) * store.k_scales[h].astype(np.float64)[:, None]
        cv = store.v_codes[h].astype(np.float64) * store.v_scales[h].astype(np.float64)[:, None]
        keys = np.concatenate([ck.reshape(-1, d), state.hot_k[:, h, :].astype(np.float64)])
        vals = np.concatenate([cv.reshape(-1, d), state.hot_v[:, h, :].astype(np.float64)])
        out[hq], lse[hq] = attend(q64[hq], keys, vals)
    return out, lse


# --------------------------------------------------------------------------- debug statistics
def quant_errors(k_hist: np.ndarray, v_hist: np.ndarray, hot_tokens: int, block_size: int,
                 quant_bits: int = 8) -> np.ndarray:
    """[n_blk, H, 2] fp64: max |x - q s| over the valid elements of every cold tile (0 for FP16 tiles)."""
    st = build_state(k_hist, v_hist, hot_tokens, block_size, quant_bits)
    k64 = np.asarray(k_hist, dtype=np.float16).astype(np.float64)
    v64 = np.asarray(v_hist, dtype=np.float16).astype(np.float64)
    err = np.zeros((st.n_blocks, st.hot_k.shape[1], 2))
    for j in range(st.n_blocks):
        nv = int(st.n_valid[j])
        for c, x in enumerate((k64, v64)):
            rows = x[j * block_size:j * block_size + nv]          # [nv, H, d]
            for h in range(err.shape[1]):
                xhat = dequantize(st.codes[j, h, c, :nv], st.scales[j, h, c])
                err[j, h, c] = float(np.max(np.abs(rows[:, h, :] - xhat))) if nv else 0.0
    return err


def attention_entropy(q: np.ndarray, state: SequenceState, sel: Optional[np.ndarray] = None) -> np.ndarray:
    """[Hq] fp64: -sum_t p_t ln p_t of each query head's softmax over the tokens decode attends (hot plus
    cold, or hot plus the selected cold tokens when sel [H, k] is given)."""
    q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
    n_q, d = q64.shape
    g = _group(n_q, state.hot_k.shape[1])
    ent = np.zeros(n_q)
    for hq in range(n_q):
        h = hq // g
        ck, _ = cold_kv(state, h)
        if sel is not None:
            ck = ck[sel[h][sel[h] >= 0]]
        keys = np.concatenate([ck, state.hot_k[:, h, :].astype(np.float64)])
        z = keys @ q64[hq] / math.sqrt(d)
        e = np.exp(z - np.max(z))
        p = e / np.sum(e)
        nz = p > 0
        ent[hq] = -float(np.sum(p[nz] * np.log(p[nz])))
    return ent


# --------------------------------------------------------------------------- metadata sizing
def header_table_bytes(total_tokens: int, hot_tokens: int, block_size: int) -> Tuple[int, int]:
    """(cold blocks, header bytes) for one sequence (Hybrid KV Cache page 5.4)."""
    _, n_cold = split_history(total_tokens, hot_tokens)
    n_blk = -(-n_cold // block_size)
    return n_blk, n_blk * HEADER_BYTES
