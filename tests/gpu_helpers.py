"""Shared helpers of the GPU parity tests: build caches from seeded inputs
through the C-ABI binding and compare them with the fp64 oracle."""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np

import oracle.hkv_oracle as orc
import workloads as wl

# Output tolerances of the fp16 attention output against the fp64 oracle.
OUT_MAX_ABS = 4e-3
OUT_MEAN_ABS = 5e-4
# log-sum-exp: fp32 logits and sums, natural log; an absolute bound well above fp32 rounding
LSE_MAX_ABS = 1e-3
# top-K: tokens whose window probability lies within this distance of the oracle's K-th value are near-ties
TOPK_TIE = 1e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def upload(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def history(w: wl.Workload, seq: int, n: int):
    return wl.tokens(w, seq, 0, n, "k"), wl.tokens(w, seq, 0, n, "v")


def fill(cache, w: wl.Workload, lens: Sequence[int], start: Optional[Sequence[int]] = None, chunk: int = 16384,
         seqs: Optional[Sequence[int]] = None) -> None:
    """Append the seeded tokens [start_b, lens_b) of every sequence, in bulk chunks."""
    B = cache.batch
    seqs = list(range(B)) if seqs is None else list(seqs)
    start = [0] * B if start is None else list(start)
    lens = list(lens)
    pos = list(start)
    while any(pos[b] < lens[b] for b in range(B)):
        cnt = max(min(chunk, lens[b] - pos[b]) for b in range(B))
        kb = np.zeros((B, cnt, w.n_kv_heads, w.head_dim), dtype=np.float16)
        vb = np.zeros_like(kb)
        n_new = np.zeros(B, dtype=np.int32)
        for b in range(B):
            take = max(0, min(cnt, lens[b] - pos[b]))
            if take:
                kb[b, :take] = wl.tokens(w, seqs[b], pos[b], take, "k")
                vb[b, :take] = wl.tokens(w, seqs[b], pos[b], take, "v")
            n_new[b] = take
            pos[b] += take
        cache.append(upload(kb), upload(vb), n_new)
    torch_mod().cuda.synchronize()


def make_cache(w: wl.Workload, max_tokens: int, batch: Optional[int] = None, phys_ids=None, num_phys: int = 0):
    import int8_kv_cache_hkv_amd as hkv
    return hkv.HybridKVCache(w.n_kv_heads, w.head_dim, batch or w.batch, max_tokens, hot_tokens=w.hot_tokens,
                             block_size=w.block_size, quant_bits=w.quant_bits, num_phys_blocks=num_phys,
                             phys_ids=phys_ids)


def check_state(cache, states: List[orc.SequenceState], seqs: Optional[Sequence[int]] = None,
                codes: Optional[np.ndarray] = None, scales: Optional[np.ndarray] = None) -> None:
    """Codes, scales, headers and the hot ring: bit-exact against the oracle states."""
    seqs = list(range(len(states))) if seqs is None else list(seqs)
    codes = cache.cold_codes() if codes is None else codes
    scales = cache.scale_array() if scales is None else scales
    hdr = cache.header_array()
    hot = cache.hot_array()
    seq_len = cache.seq_len.cpu().numpy()
    for b, st in zip(seqs, states):
        assert int(seq_len[b]) == st.n_tokens == int(cache.seq_len_host[b]), (b, seq_len[b], st.n_tokens)
        for j in range(st.n_blocks):
            phys = int(hdr[b, j, 0])
            nv = int(st.n_valid[j])
            assert int(hdr[b, j, 1]) == nv and int(hdr[b, j, 2]) == j, (b, j, hdr[b, j])
            got = codes[phys]
            want = st.codes[j]
            if got.dtype == np.float16:  # an FP16 cold zone: compare bit patterns
                got, want = got.view(np.uint16), np.asarray(want, dtype=np.float16).view(np.uint16)
            if not np.array_equal(got[:, :, :nv], want[:, :, :nv]):
                bad = np.argwhere(got[:, :, :nv] != want[:, :, :nv])
                raise AssertionError(f"seq {b} block {j}: {len(bad)} code mismatches, first {bad[:3].tolist()}")
            assert not got[:, :, nv:].any(), f"seq {b} block {j}: rows past n_valid are not zero"
            sg, sw = scales[phys], st.scales[j]
            assert np.array_equal(sg.view(np.uint32), sw.view(np.uint32)), (b, j, sg, sw)
        n_hot = st.n_hot
        for i in range(n_hot):
            p = st.n_tokens - n_hot + i
            slot = p % cache.T
            assert np.array_equal(hot[b, :, slot, 0].view(np.uint16), st.hot_k[i].view(np.uint16)), (b, p)
            assert np.array_equal(hot[b, :, slot, 1].view(np.uint16), st.hot_v[i].view(np.uint16)), (b, p)


def compare_out(got: np.ndarray, want: np.ndarray, what: str) -> dict:
    diff = np.abs(got.astype(np.float64) - want)
    mx, mean = float(diff.max()), float(diff.mean())
    log(f"  {what}: max|d|={mx:.3e} mean|d|={mean:.3e}")
    assert np.all(np.isfinite(got)), what
    assert mx <= OUT_MAX_ABS, f"{what}: max abs {mx}"
    assert mean <= OUT_MEAN_ABS, f"{what}: mean abs {mean}"
    return {"max": mx, "mean": mean}


def compare_lse(got: np.ndarray, want: np.ndarray, what: str) -> None:
    d = float(np.max(np.abs(got.astype(np.float64) - want)))
    assert d <= LSE_MAX_ABS, f"{what}: lse max abs {d}"


def compare_topk(got: np.ndarray, want: np.ndarray, p: np.ndarray, tau: float, n_cold: int, k: int, what: str):
    """Index sets equal once near-ties of the K-th probability are removed; the rest must be valid."""
    g = got[got >= 0]
    assert np.all(np.diff(g) > 0), f"{what}: not ascending / duplicates"
    assert np.all(got[len(g):] == -1) and len(g) == min(k, n_cold), f"{what}: padding"
    assert np.all(g < n_cold)
    if n_cold <= k:
        assert np.array_equal(g, np.arange(n_cold)), what
        return
    near = set(np.nonzero(np.abs(p - tau) <= TOPK_TIE)[0].tolist())
    gs = set(g.tolist()) - near
    ws = set(want[want >= 0].tolist()) - near
    assert gs == ws, f"{what}: {len(gs ^ ws)} differing indices outside near-ties"
