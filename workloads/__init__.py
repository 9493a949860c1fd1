"""Seeded synthetic inputs for the hybrid FP16/INT8 KV-cache decode path.

This module only draws random inputs (token keys/values, decode queries,
sequence lengths, physical-block placements). It contains none of the
method's arithmetic, so the CPU oracle and the GPU path can both consume the
exact same host fp16 bytes without sharing any computation.

Every draw is keyed by ``numpy.random.SeedSequence([BASE_SEED, config index,
kind, sequence, chunk])`` so that any 64-token chunk of any sequence can be
regenerated on its own (the oracle re-derives only the sequences it checks).
Values are drawn as float32 N(0, 1) and cast to fp16 with round-to-nearest-even.

Workload shapes follow the five decode configurations the cache is measured
on (tiny correctness case, a Llama-3-8B-shaped layer, a ragged paged batch,
a 131072-token context and a top-K sparse case).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, List, Optional

import numpy as np

BASE_SEED = 20261202
CHUNK = 64  # tokens per independently seeded chunk (independent of the cache block size)

KIND_K, KIND_V, KIND_Q, KIND_LEN, KIND_PERM, KIND_OUTLIER = 0, 1, 2, 3, 4, 5


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int
    batch: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    context: int = 0                 # tokens per sequence at decode time (uniform configs)
    hot_tokens: int = 32
    block_size: int = 64
    quant_bits: int = 8
    outlier_channels: int = 0        # K channels per kv-head scaled up (shared by all tokens)
    outlier_scale: float = 1.0
    len_lo: int = 0                  # ragged: inclusive length range
    len_hi: int = 0
    steps: int = 1                   # ragged: append+decode steps
    permuted_blocks: bool = False    # physical block ids at a seeded permutation
    k_sel: int = 0                   # top-K budget

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 0, batch=1, n_kv_heads=2, n_q_heads=4, head_dim=64, context=288),
    "llama8b": Workload("llama8b", 1, batch=8, n_kv_heads=8, n_q_heads=32, head_dim=128, context=2048,
                        outlier_channels=4, outlier_scale=10.0),
    "ragged": Workload("ragged", 2, batch=64, n_kv_heads=8, n_q_heads=32, head_dim=128,
                       len_lo=128, len_hi=8192, steps=64, permuted_blocks=True),
    "long": Workload("long", 3, batch=4, n_kv_heads=8, n_q_heads=32, head_dim=128, context=131072),
    "topk": Workload("topk", 4, batch=16, n_kv_heads=8, n_q_heads=32, head_dim=128, context=32768, k_sel=512),
}


def _rng(w: Workload, kind: int, seq: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, w.index, kind, seq, chunk])))


def outlier_channel_ids(w: Workload) -> np.ndarray:
    """[n_kv_heads, outlier_channels] channel indices, drawn once per kv-head."""
    if w.outlier_channels == 0:
        return np.zeros((w.n_kv_heads, 0), dtype=np.int64)
    out = np.empty((w.n_kv_heads, w.outlier_channels), dtype=np.int64)
    for h in range(w.n_kv_heads):
        out[h] = _rng(w, KIND_OUTLIER, 0, h).choice(w.head_dim, size=w.outlier_channels, replace=False)
    return out


def _chunk(w: Workload, kind: int, seq: int, chunk: int, outl: Optional[np.ndarray]) -> np.ndarray:
    x = _rng(w, kind, seq, chunk).standard_normal((CHUNK, w.n_kv_heads, w.head_dim), dtype=np.float32)
    if kind == KIND_K and outl is not None and outl.shape[1] > 0:
        for h in range(w.n_kv_heads):
            x[:, h, outl[h]] *= np.float32(w.outlier_scale)
    return x.astype(np.float16)


def tokens(w: Workload, seq: int, start: int, count: int, kind: str) -> np.ndarray:
    """fp16 [count, n_kv_heads, head_dim] keys ('k') or values ('v') for positions [start, start+count)."""
    kcode = KIND_K if kind == "k" else KIND_V
    outl = outlier_channel_ids(w) if kcode == KIND_K else None
    out = np.empty((count, w.n_kv_heads, w.head_dim), dtype=np.float16)
    if count == 0:
        return out
    c0, c1 = start // CHUNK, (start + count - 1) // CHUNK
    for c in range(c0, c1 + 1):
        blk = _chunk(w, kcode, seq, c, outl)
        lo = max(start, c * CHUNK)
        hi = min(start + count, (c + 1) * CHUNK)
        out[lo - start:hi - start] = blk[lo - c * CHUNK:hi - c * CHUNK]
    return out


def batch_tokens(w: Workload, seqs: List[int], start: int, count: int, kind: str,
                 threads: Optional[int] = None) -> np.ndarray:
    """fp16 [len(seqs), count, H, d], generated in parallel over sequences."""
    out = np.empty((len(seqs), count, w.n_kv_heads, w.head_dim), dtype=np.float16)
    nthr = threads or min(16, os.cpu_count() or 1)

    def one(i: int) -> None:
        out[i] = tokens(w, seqs[i], start, count, kind)

    with _cf.ThreadPoolExecutor(max_workers=nthr) as ex:
        list(ex.map(one, range(len(seqs))))
    return out


def query(w: Workload, seq: int, step: int = 0) -> np.ndarray:
    """fp16 [n_q_heads, head_dim] decode query of sequence ``seq`` at decode step ``step``."""
    x = _rng(w, KIND_Q, seq, step).standard_normal((w.n_q_heads, w.head_dim), dtype=np.float32)
    return x.astype(np.float16)


def queries(w: Workload, step: int = 0) -> np.ndarray:
    return np.stack([query(w, b, step) for b in range(w.batch)])


def lengths(w: Workload) -> np.ndarray:
    """int64 [batch] initial context lengths (uniform configs: all equal to ``context``)."""
    if w.len_hi > 0:
        return _rng(w, KIND_LEN, 0, 0).integers(w.len_lo, w.len_hi, size=w.batch, endpoint=True)
    return np.full(w.batch, w.context, dtype=np.int64)


def block_permutation(w: Workload, n_phys: int) -> np.ndarray:
    """Physical block ids for the logical blocks, in (sequence, logical block) order."""
    if not w.permuted_blocks:
        return np.arange(n_phys, dtype=np.int64)
    return _rng(w, KIND_PERM, 0, 0).permutation(n_phys)

