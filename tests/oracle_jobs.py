"""Oracle work items for the full-size parity tests, run in spawned worker
processes (numpy only: no torch, no HIP) so that several sequences of the
131072-token and 32768-token workloads are checked in parallel.

Every function regenerates its sequence's seeded history itself (the inputs
module holds no arithmetic of the method) and calls only the fp64 oracle.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import multiprocessing as mp
import os
from typing import Dict, Optional

import numpy as np

import oracle.hkv_oracle as orc
import workloads as wl


def pool(n_jobs: int) -> cf.ProcessPoolExecutor:
    """A spawn-started process pool (never forked from a process that may hold a GPU context)."""
    workers = max(1, min(n_jobs, 8, os.cpu_count() or 1))
    return cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))


def _workload(name: str, overrides: Optional[Dict] = None) -> wl.Workload:
    w = wl.WORKLOADS[name]
    return dataclasses.replace(w, **overrides) if overrides else w


def state_of(name: str, seq: int, n: int, overrides: Optional[Dict] = None) -> orc.SequenceState:
    """Oracle cache state of sequence `seq` after its first n seeded tokens."""
    w = _workload(name, overrides)
    k = wl.tokens(w, seq, 0, n, "k")
    v = wl.tokens(w, seq, 0, n, "v")
    return orc.build_state(k, v, w.hot_tokens, w.block_size, w.quant_bits)


def decode_job(name: str, seq: int, lengths, queries, with_state_at: int = -1,
               overrides: Optional[Dict] = None):
    """Dense decode of one sequence at each length in `lengths` with the matching query [Hq, d];
    returns [(out, lse)] and, when with_state_at >= 0, the oracle state at that length."""
    w = _workload(name, overrides)
    n_max = max(lengths)
    k = wl.tokens(w, seq, 0, n_max, "k")
    v = wl.tokens(w, seq, 0, n_max, "v")
    res = []
    keep = None
    for n, q in zip(lengths, queries):
        st = orc.build_state(k[:n], v[:n], w.hot_tokens, w.block_size, w.quant_bits)
        res.append(orc.decode(q, st))
        if n == with_state_at:
            keep = st
    return res, keep


def topk_job(name: str, seq: int, q: np.ndarray, k_sel: int, gpu_idx: np.ndarray,
             overrides: Optional[Dict] = None):
    """Top-K selection of one sequence (index sets, window probabilities, K-th value per kv-head) and
    the sparse decode over the selection the GPU returned (gpu_idx [H, k])."""
    w = _workload(name, overrides)
    st = state_of(name, seq, w.context, overrides)
    idx, p, tau = orc.topk_select(q, st, k_sel)
    o_ref, l_ref = orc.sparse_decode(q, st, gpu_idx)
    return idx, p, tau, st.n_cold, o_ref, l_ref
