#!/usr/bin/env python3
"""Benchmark of the hybrid FP16/INT8 KV-cache decode path on one MI355X.

One step = one decode step of a Llama-3-8B-shaped layer (batch 8, 32 query /
8 kv heads, head_dim 128, 2048 cached tokens = 32 FP16 hot + 31 full INT8
blocks + 1 half block): one new token appended per sequence (spill +
re-quantisation of the touched cold block) and the dense decode, issued as one
fused launch (hkv_append_decode).  Steps rotate over independent cache
instances whose combined size exceeds the 256 MB Infinity Cache, so every step
streams its cache from HBM.

Printed: one JSON line.  `value` = algorithmic bytes per step / step time (GB/s,
median of --trials trials of --steps steps, host clock with device
synchronisation around each trial).  Every leg carries a `roofline` block for
its dominant launch: algorithmic bytes per launch / the launch's average
duration, from a HIP event pair on the launch stream around each timed trial
(median over trials).  After its timed trials every leg recomputes its last
output outside the timed region (and, where it is cheap, with the fp64
oracle) and the run exits with status 3 if any check fails.

Legs (`--leg`, default all): llama8b (the headline step), separate (the same
step as hkv_append + hkv_decode_attn), long (131072 tokens), llama8b_int4 /
long_int4 / llama8b_fp16 / long_fp16 (the same steps with 4-bit cold blocks or
an FP16 cold zone), sparse (top-K
selection + sparse decode, 32768 tokens), ragged (64 sequences of seeded
lengths), phases (per-workgroup timestamps of one llama8b step, and of the same
step at 544 tokens), graph (the llama8b step from a HIP graph), read_floor (a
plain one-launch read of the llama8b step's bytes), cpu (the fp64 oracle on the
host).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn KV GB/s (% of HBM peak) + decode queries/sec, hybrid INT8/FP16"
OUT_MAX_ABS, OUT_MEAN_ABS = 4e-3, 5e-4

# HBM bytes per launch from hardware counters (FETCH_SIZE x 2.000 + WRITE_SIZE x 1.000 KiB per
# dispatch; the factors make a 256 MiB elementwise copy read and write exactly its size), recorded
# in the profiles folder (path_kernels_hbm_traffic.md).  A figure holds only for the kernel sources
# of its leg (TRAFFIC_SOURCES) as they were when it was taken: it is reported as null once their code
# changes (the hash skips comments and blank lines).
COUNTER_TRAFFIC = {
    "sources_sha256": {"llama8b": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "long": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "llama8b_b4": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "long_b4": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "llama8b_b0": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "long_b0": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "topk": "50c5488395d960e412301b4c1437395ed0ad831d7515fe9742b634d8447e46ba", "sparse_decode": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "store_decode": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "compact": "686c662f52804052b365258c44024bfc6152993b907378f690db7ca034320f82", "ragged": "ce513c169f5d26665ef634db6d2cfcab71d71aeaf13ee1decc28b485084381cf", "prefill_llama8b_2048": "111c6b7ed0010d05675ad083b3e02f035479898bf9d2db802e381cb06d306165", "prefill_topk_8192": "111c6b7ed0010d05675ad083b3e02f035479898bf9d2db802e381cb06d306165"},
    "bytes_per_launch": {"llama8b": 36966974, "long": 1084441620, "llama8b_b4": 20697825, "long_b4": 550152559, "llama8b_b0": 69420191, "long_b0": 2157510913, "topk": 562830430, "sparse_decode": 190040815, "store_decode": 21981696, "compact": 197185291, "ragged": 614900311, "prefill_llama8b_2048": 104263607, "prefill_topk_8192": 813429376},
}
DECODE_SOURCES = ("decode_impl.h", "decode_inst.hip", "hkv_device.h", "hkv_internal.h")
TRAFFIC_SOURCES = {"topk": ("topk.hip", "hkv_device.h", "hkv_internal.h"),
                   "compact": ("compact.hip", "hkv_device.h", "hkv_internal.h"),
                   "prefill_llama8b_2048": ("append.hip", "hkv_device.h", "hkv_internal.h"),
                   "prefill_topk_8192": ("append.hip", "hkv_device.h", "hkv_internal.h")}  # every other leg: the decode's


def leg_sources(leg: str):
    return TRAFFIC_SOURCES.get(leg, DECODE_SOURCES)


def code_text(src: str) -> str:
    """Source text without // and /* */ comments, leading/trailing blanks and empty lines."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).strip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln)


def sources_hash(files=DECODE_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        p = os.path.join(ROOT, "int8_kv_cache_hkv_amd", "csrc", f)
        if os.path.exists(p):
            with open(p, encoding="utf-8") as fh:
                h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def counter_traffic(leg: str):
    """(bytes per launch, source) recorded from the counters for this leg, or (None, reason)."""
    if (leg not in COUNTER_TRAFFIC["bytes_per_launch"]
            or COUNTER_TRAFFIC["sources_sha256"].get(leg) != sources_hash(leg_sources(leg))):
        return None, "not measured on the current kernel sources"
    return COUNTER_TRAFFIC["bytes_per_launch"][leg], "recorded from rocprofv3 FETCH_SIZE/WRITE_SIZE (profiles folder)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic bytes
def cold_elem_bytes(bits=8):
    """Bytes per cold element: an 8-bit code, a 4-bit code, or an fp16 value (quant_bits 0)."""
    return {8: 1.0, 4: 0.5, 0: 2.0}[bits]


def decode_bytes(n, H, Hq, d, T=32, S=64, with_out=True, bits=8):
    """Bytes the dense decode must move for one sequence of n cached tokens: the K and V codes (or fp16
    values) of the cold tokens, the two fp32 scales per cold block and kv-head, the 16-byte headers,
    the fp16 hot tokens, the fp16 query (and the fp16 output)."""
    n_hot = min(n, T)
    n_cold = n - n_hot
    n_blk = -(-n_cold // S)
    b = 2 * n_cold * H * d * cold_elem_bytes(bits) + 8 * n_blk * H + 16 * n_blk + 4 * n_hot * H * d + 2 * Hq * d
    return int(b + (2 * Hq * d if with_out else 0))


def append_bytes(n_new_tokens, H, d, bits=8):
    """Per appended token once the hot zone is full: read K,V (4Hd), write the ring slot (4Hd),
    read the spilled token (4Hd), write its codes (2Hd x element bytes), write the tail shadow (4Hd),
    scales + header."""
    return int(n_new_tokens * ((16 + 2 * cold_elem_bytes(bits)) * H * d + 8 * H + 16))


def sparse_bytes(n, H, Hq, d, k, T=32):
    """Sparse decode of one sequence: the selected tokens' int8 K and V codes and their blocks' scales
    and headers, the hot zone, q in / out, the selection read."""
    n_hot = min(n, T)
    sel = min(k, n - n_hot)
    return 2 * sel * H * d + 8 * sel * H + 16 * sel + 4 * n_hot * H * d + 4 * Hq * d + 4 * H * k


def store_decode_bytes(n, H, Hq, d, k, T=32):
    """Decode over a compacted sparse store of one sequence: the stored tokens' int8 K and V codes and
    their own scales, the counts, the hot zone, q in / out."""
    n_hot = min(n, T)
    sel = min(k, n - n_hot)
    return 2 * sel * H * d + 8 * sel * H + 4 * H + 4 * n_hot * H * d + 4 * Hq * d


def compact_bytes(n, H, d, k, T=32):
    """Building the compacted store of one sequence: read the selection and the selected tokens' headers,
    codes and scales, write the codes, scales and counts."""
    sel = min(k, n - min(n, T))
    return 4 * H * k + 16 * sel * H + 2 * (2 * sel * H * d + 8 * sel * H) + 4 * H


def topk_bytes(n, H, Hq, d, k, T=32):
    """Top-K selection of one sequence: the int8 K codes of the cold tokens (the scale cancels in a
    cosine), the headers, the query and the index list written."""
    n_cold = n - min(n, T)
    return n_cold * H * d + 16 * (-(-n_cold // 64)) + 2 * Hq * d + 4 * H * k


def roofline(kernel, nbytes, ms, leg):
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic, src = counter_traffic(leg)
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_source": src,
            "bytes_per_launch": int(nbytes), "avg_launch_ms": round(ms, 6)}


# ----------------------------------------------------------------------------- timing
def timed_trials(torch, step, first, steps, trials, preroll=4):
    """Host-clock trials: `trials` trials of exactly `steps` calls step(i) (i counts on from
    `first`), each bracketed by torch.cuda.synchronize() on both sides.  Then as many device-timed
    trials: `preroll` untimed calls are queued first so that the GPU is busy when the first timed
    launch is issued, and an event pair recorded on the current stream (the stream every launch
    goes to) brackets the `steps` timed calls, so the device interval is back-to-back launches only.
    Returns the medians (host ms per step, device ms per launch-step), every trial's figures and the
    values step() returned in the host-clock trials."""
    host, dev, rets = [], [], []
    i = first
    for _ in range(trials):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            rets.append(step(i))
            i += 1
        torch.cuda.synchronize()
        host.append((time.perf_counter() - t0) * 1e3 / steps)
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        for _ in range(preroll):
            step(i)
            i += 1
        e0.record()
        for _ in range(steps):
            step(i)
            i += 1
        e1.record()
        torch.cuda.synchronize()
        dev.append(e0.elapsed_time(e1) / steps)
    return {"ms_per_step": statistics.median(host), "device_ms_per_step": statistics.median(dev),
            "trials_ms": [round(x, 6) for x in host], "trials_device_ms": [round(x, 6) for x in dev],
            "next": i, "rets": rets}


def timed_calls(trials, steps, preroll=4):
    """Calls of step() that timed_trials makes."""
    return trials * (2 * steps + preroll)


def out_close(got, want, what):
    """Max / mean absolute difference of two fp16 outputs against the bench's tolerance."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    ok = bool(np.all(np.isfinite(got)) and d.max() <= OUT_MAX_ABS and d.mean() <= OUT_MEAN_ABS)
    return {"what": what, "max_abs": float(d.max()), "mean_abs": float(d.mean()), "ok": ok}


CHECKS = []


def record_check(c):
    CHECKS.append(c)
    if not c["ok"]:
        log(f"SELF-CHECK FAILED: {c}")


# ----------------------------------------------------------------------------- legs
class Inst:
    """One cache instance plus pre-marshalled C-ABI arguments."""

    def __init__(self, hkv, w, cap_tokens, quant_bits=8):
        self.c = hkv.HybridKVCache(w.n_kv_heads, w.head_dim, w.batch, cap_tokens, quant_bits=quant_bits)
        self.desc_ref = ctypes.byref(self.c.desc)


def decode_step_leg(hkv, torch, w, n0, steps, warmup, trials, R, label, fused=True, quant_bits=8,
                    oracle_check=True):
    """Rotating-instance decode steps of a uniform-length workload: one hkv_append_decode launch per
    step (fused) or hkv_append then hkv_decode_attn.  Returns timing, bytes and the self-check."""
    import workloads as wl
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    total = warmup + timed_calls(trials, steps)
    uses = -(-total // R) + 1
    cap = n0 + uses + 1
    log(f"{label}: {R} instances of B={B} n0={n0} (cap {cap}), generating inputs")
    insts = [Inst(hkv, w, cap, quant_bits) for _ in range(R)]
    chunk = 16384
    for s in range(0, n0, chunk):
        cnt = min(chunk, n0 - s)
        kh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s, cnt, "k")).cuda()
        vh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s, cnt, "v")).cuda()
        for it in insts:
            it.c.append(kh, vh)
        del kh, vh
    torch.cuda.synchronize()
    newk = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, uses, "k")).cuda()   # [B, uses, H, d]
    newv = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, uses, "v")).cuda()
    newk_u = [newk[:, u].contiguous() for u in range(uses)]
    newv_u = [newv[:, u].contiguous() for u in range(uses)]
    NQ = 32
    qs = [torch.from_numpy(wl.queries(w, step=i)).cuda() for i in range(NQ)]
    out = torch.empty_like(qs[0])
    ws = insts[0].c.workspace(Hq)
    ws_ptr, ws_len = ws.data_ptr(), ws.numel()
    ones = np.ones(B, dtype=np.int32)
    stream = torch.cuda.current_stream().cuda_stream
    lib = hkv._lib
    used = [0] * R

    def step(i):
        r = i % R
        it = insts[r]
        u = used[r]
        if fused:
            st = lib.hkv_append_decode(it.c.handle, it.desc_ref, newk_u[u].data_ptr(), newv_u[u].data_ptr(),
                                       qs[i % NQ].data_ptr(), Hq, out.data_ptr(), None, ws_ptr, ws_len, stream)
        else:
            st = lib.hkv_append(it.c.handle, it.desc_ref, newk_u[u].data_ptr(), newv_u[u].data_ptr(),
                                ones.ctypes.data, 1, stream)
            if not st:
                st = lib.hkv_decode_attn(it.c.handle, it.desc_ref, qs[i % NQ].data_ptr(), Hq, None, 0,
                                         out.data_ptr(), None, ws_ptr, ws_len, stream)
        if st:
            raise hkv.HKVError(st, label)
        used[r] += 1
        return n0 + used[r]   # cached length after the step

    for i in range(warmup):
        step(i)
    res = timed_trials(torch, step, warmup, steps, trials)
    lens = res.pop("rets")
    step_bytes = [B * (decode_bytes(n, H, Hq, d, bits=quant_bits) + append_bytes(1, H, d, quant_bits)) for n in lens]
    kern_bytes = step_bytes if fused else [B * decode_bytes(n, H, Hq, d, bits=quant_bits) for n in lens]
    # ---- self-check of the last timed step, outside the timed region
    last = res["next"] - 1
    r_last, q_last = last % R, qs[last % NQ]
    n_last = n0 + used[r_last]
    got = out.cpu().numpy()
    chk = torch.empty_like(q_last)
    it = insts[r_last]
    st = lib.hkv_decode_attn(it.c.handle, it.desc_ref, q_last.data_ptr(), Hq, None, 0, chk.data_ptr(), None,
                             ws_ptr, ws_len, stream)
    if st:
        raise hkv.HKVError(st, "self-check decode")
    torch.cuda.synchronize()
    record_check(out_close(got, chk.cpu().numpy(), f"{label}: last timed output vs hkv_decode_attn recompute"))
    if oracle_check:
        import oracle.hkv_oracle as orc
        k = wl.tokens(w, 0, 0, n_last, "k")
        v = wl.tokens(w, 0, 0, n_last, "v")
        o_ref, _ = orc.decode(q_last.cpu().numpy()[0], orc.build_state(k, v, w.hot_tokens, w.block_size, quant_bits))
        record_check(out_close(got[0], o_ref, f"{label}: last timed output, sequence 0, vs the fp64 oracle"))
    for it in insts:
        it.c.close()
    del insts
    torch.cuda.empty_cache()
    res["bytes_per_step"] = statistics.mean(step_bytes)
    res["kernel_bytes_per_step"] = statistics.mean(kern_bytes)
    res["gbs"] = res["bytes_per_step"] / (res["ms_per_step"] * 1e-3) / 1e9
    return res


def leg_llama8b(hkv, torch, args):
    import workloads as wl
    w = wl.WORKLOADS["llama8b"]
    r = decode_step_leg(hkv, torch, w, w.context - 1, args.steps, args.warmup, args.trials, args.instances,
                        "llama8b")
    return w, r


def leg_separate(hkv, torch, args):
    import workloads as wl
    w = wl.WORKLOADS["llama8b"]
    r = decode_step_leg(hkv, torch, w, w.context - 1, args.steps, args.warmup, args.trials, args.instances,
                        "llama8b (separate calls)", fused=False)
    return {"what": "the llama8b step as hkv_append then hkv_decode_attn (two launches per step)",
            "ms_per_step": r["ms_per_step"], "trials_ms": r["trials_ms"], "gbs": r["gbs"],
            "pct_hbm_peak": 100 * r["gbs"] / HBM_PEAK_GBS}


def long_steps(args):
    """Steps per trial (and untimed warm-up steps) of the 131072-token legs: 4x --steps, 16 to 64.
    A host-clock trial starts from an idle GPU (synchronize), so its first launches run before the
    clock has settled; 64 steps (7 to 21 ms) keep that ramp to a small part of the trial.  The 4-bit
    step, bound by its instruction stream, shows it most: 16-step trials of 106 to 145 us against
    102 us back-to-back."""
    return max(16, min(4 * args.steps, 64))


def leg_long(hkv, torch, args):
    import workloads as wl
    w = wl.WORKLOADS["long"]
    steps = long_steps(args)
    r = decode_step_leg(hkv, torch, w, w.context - 1, steps, steps, args.trials, 2, "long", oracle_check=False)
    return {"workload": "long: B=4, 131072 tokens, 32/8 heads, d=128, step = fused append 1 token + decode",
            "steps": steps, "ms_per_step": r["ms_per_step"], "trials_ms": r["trials_ms"], "gbs": r["gbs"],
            "pct_hbm_peak": 100 * r["gbs"] / HBM_PEAK_GBS,
            "roofline": roofline("decode_kernel (fused append + decode, claim walk)", r["kernel_bytes_per_step"],
                                 r["device_ms_per_step"], "long")}


def leg_width(hkv, torch, args, name, bits):
    """The llama8b step or the 131072-token step with 4-bit cold blocks or an FP16 cold zone (Hybrid KV
    Cache page 3.1: quantization_bits 4; 5.2: quantization_bits 0)."""
    import workloads as wl
    w = wl.WORKLOADS[name]
    if name == "long":
        steps, warmup, R, check = long_steps(args), long_steps(args), 2, False
    else:
        steps, warmup, R, check = args.steps, args.warmup, args.instances, True
    label = f"{name} {'fp16' if bits == 0 else str(bits) + '-bit'} cold"
    r = decode_step_leg(hkv, torch, w, w.context - 1, steps, warmup, args.trials, R, label, quant_bits=bits,
                        oracle_check=check)
    ms = r["ms_per_step"]
    return {"workload": f"{name} workload, quant_bits {bits}, step = fused append 1 token + decode", "steps": steps,
            "ms_per_step": ms, "trials_ms": r["trials_ms"], "gbs": r["gbs"],
            "pct_hbm_peak": 100 * r["gbs"] / HBM_PEAK_GBS,
            "queries_per_s": w.batch / (ms * 1e-3), "head_queries_per_s": w.batch * w.n_q_heads / (ms * 1e-3),
            "roofline": roofline(f"decode_kernel (fused append + decode, {label})", r["kernel_bytes_per_step"],
                                 r["device_ms_per_step"], f"{name}_b{bits}")}


def leg_sparse(hkv, torch, args):
    """Top-K selection + sparse decode of the 32768-token workload, alternating two instances."""
    import workloads as wl
    w = wl.WORKLOADS["topk"]
    B, H, Hq, d, k = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim, w.k_sel
    n = w.context
    steps = max(8, min(args.steps, 20))
    log(f"sparse: 2 instances of B={B} n={n}, K={k}")
    insts = [hkv.HybridKVCache(H, d, B, n) for _ in range(2)]
    chunk = 8192
    for s in range(0, n, chunk):
        kh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s, chunk, "k")).cuda()
        vh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s, chunk, "v")).cuda()
        for c in insts:
            c.append(kh, vh)
        del kh, vh
    q = torch.from_numpy(wl.queries(w)).cuda()
    out = torch.empty_like(q)
    idx = torch.empty((B, H, k), dtype=torch.int32, device="cuda")
    ws = insts[0].workspace(Hq, k)
    for c in insts:
        c.topk(q, k, out_idx=idx, workspace=ws)
        c.decode(q, out=out, sel_idx=idx, k_sel=k, workspace=ws)
    torch.cuda.synchronize()

    def topk_only(i):
        insts[i % 2].topk(q, k, out_idx=idx, workspace=ws)

    def sparse_only(i):
        insts[i % 2].decode(q, out=out, sel_idx=idx, k_sel=k, workspace=ws)

    def both(i):
        topk_only(i)
        sparse_only(i)

    stores = [c.sparse_store(idx, k) for c in insts]
    out_st = torch.empty_like(q)

    def compact_only(i):
        insts[i % 2].sparse_store(idx, k, store=stores[i % 2])

    def store_only(i):
        insts[i % 2].decode_store(q, stores[i % 2], k, out=out_st, workspace=ws)

    def select_compact_decode(i):
        topk_only(i)
        compact_only(i)
        store_only(i)

    for i in range(steps):  # untimed: the clock settles before the first host-clock trial
        both(i)
    res = timed_trials(torch, both, 0, steps, args.trials)
    t_topk = timed_trials(torch, topk_only, 0, steps, args.trials)
    t_sparse = timed_trials(torch, sparse_only, 0, steps, args.trials)
    res_c = timed_trials(torch, select_compact_decode, 0, steps, args.trials)
    t_compact = timed_trials(torch, compact_only, 0, steps, args.trials)
    t_store = timed_trials(torch, store_only, 0, steps, args.trials)
    torch.cuda.synchronize()
    record_check(out_close(out_st.cpu().numpy(), out.cpu().numpy(),
                           "sparse: decode over the compacted store vs the gather decode of the same selection"))
    # self-check: the last step's selection and output recomputed, then the oracle on sequence 0
    c_last = insts[(res["next"] - 1) % 2]
    idx_last, out_last = idx.cpu().numpy(), out.cpu().numpy()
    idx2 = torch.empty_like(idx)
    out2 = torch.empty_like(out)
    c_last.topk(q, k, out_idx=idx2, workspace=ws)
    c_last.decode(q, out=out2, sel_idx=idx2, k_sel=k, workspace=ws)
    torch.cuda.synchronize()
    same = bool(np.array_equal(idx2.cpu().numpy(), idx_last))
    record_check({"what": "sparse: last timed selection vs recompute (bitwise)", "ok": same})
    record_check(out_close(out_last, out2.cpu().numpy(), "sparse: last timed output vs recompute"))
    import oracle.hkv_oracle as orc
    kk = wl.tokens(w, 0, 0, n, "k")
    vv = wl.tokens(w, 0, 0, n, "v")
    st = orc.build_state(kk, vv, w.hot_tokens, w.block_size)
    want, p, tau = orc.topk_select(wl.queries(w)[0], st, k)
    ok = True
    for h in range(H):
        near = set(np.nonzero(np.abs(p[h] - tau[h]) <= 1e-5)[0].tolist())
        ok &= (set(idx_last[0, h].tolist()) - near) == (set(want[h].tolist()) - near)
    record_check({"what": "sparse: last timed selection, sequence 0, vs the fp64 oracle (outside near-ties)",
                  "ok": bool(ok)})
    o_ref, _ = orc.sparse_decode(wl.queries(w)[0], st, idx_last[0])
    record_check(out_close(out_last[0], o_ref, "sparse: last timed output, sequence 0, vs the fp64 oracle"))
    # per-kernel split of the selection (score vs select) from dispatch-recorded events, untimed pass
    for c in insts:
        hkv.hkv_timing_enable(c.handle, True)
    for i in range(steps):
        both(i)
    torch.cuda.synchronize()
    km = {}
    for kname in ("topk_score", "topk_select", "decode_sparse"):
        tot, cnt = 0.0, 0
        for c in insts:
            a, b = hkv.hkv_timing_read(c.handle, kname, reset=True)
            tot, cnt = tot + a, cnt + b
        km[kname] = tot / cnt if cnt else None
    for c in insts:
        hkv.hkv_timing_enable(c.handle, False)
        c.close()
    del insts
    torch.cuda.empty_cache()
    tb = B * topk_bytes(n, H, Hq, d, k)
    sb = B * sparse_bytes(n, H, Hq, d, k)
    stb = B * store_decode_bytes(n, H, Hq, d, k)
    cb = B * compact_bytes(n, H, d, k)
    return {"workload": "topk: B=16, 32768 tokens, 32/8 heads, d=128, K=512; step = hkv_topk_select + sparse "
                        "hkv_decode_attn", "steps": steps,
            "ms_per_step": res["ms_per_step"], "trials_ms": res["trials_ms"],
            "gbs": (tb + sb) / (res["ms_per_step"] * 1e-3) / 1e9,
            "pct_hbm_peak": 100 * (tb + sb) / (res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "roofline": roofline("topk_score_kernel + topk_select_kernel (one hkv_topk_select call)", tb,
                                 t_topk["device_ms_per_step"], "topk"),
            "roofline_sparse_decode": roofline("decode_kernel, sparse (gathered tokens)", sb,
                                               t_sparse["device_ms_per_step"], "sparse_decode"),
            "compacted_store": {
                "what": "KV Cache reuse page 2: the selected tokens re-packed into a compacted store "
                        "(hkv_sparse_compact), decoded from it (hkv_decode_attn_compact)",
                "ms_per_step_select_compact_decode": res_c["ms_per_step"],
                "trials_ms": res_c["trials_ms"],
                "roofline_store_decode": roofline("decode_kernel, compacted store units", stb,
                                                  t_store["device_ms_per_step"], "store_decode"),
                "roofline_compact": roofline("sparse_compact_kernel (gathers the selection)", cb,
                                             t_compact["device_ms_per_step"], "compact")},
            "dispatch_event_ms": km}


def leg_ragged(hkv, torch, args, steps=64, R=4, warmup=64):
    """The ragged paged batch: 64 sequences of seeded lengths in [128, 8192], cold blocks at a seeded
    permutation of the physical pool, decode steps of one appended token per sequence plus a dense
    decode (fused launch), rotating over R instances."""
    import workloads as wl
    w = wl.WORKLOADS["ragged"]
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    lens0 = [int(x) for x in wl.lengths(w)]
    trials = args.trials
    per_inst = -(-(warmup + timed_calls(trials, steps)) // R) + 2
    cap = max(lens0) + per_inst + 1
    mb = -(-(cap - w.hot_tokens) // w.block_size)
    perm = wl.block_permutation(w, B * mb).reshape(B, mb)
    log(f"ragged: {R} instances of B={B}, lengths {min(lens0)}..{max(lens0)} (cap {cap}), generating inputs")
    insts = [hkv.HybridKVCache(H, d, B, cap, phys_ids=perm) for _ in range(R)]
    chunk = 2048
    for s0 in range(0, max(lens0), chunk):
        cnt = min(chunk, max(lens0) - s0)
        kb = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s0, cnt, "k")).cuda()
        vb = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s0, cnt, "v")).cuda()
        n_new = np.array([max(0, min(cnt, n - s0)) for n in lens0], dtype=np.int32)
        for c in insts:
            c.append(kb, vb, n_new)
        del kb, vb
    torch.cuda.synchronize()
    newk = [torch.from_numpy(np.stack([wl.tokens(w, b, lens0[b] + u, 1, "k")[0] for b in range(B)])).cuda()
            for u in range(per_inst)]
    newv = [torch.from_numpy(np.stack([wl.tokens(w, b, lens0[b] + u, 1, "v")[0] for b in range(B)])).cuda()
            for u in range(per_inst)]
    qs = [torch.from_numpy(wl.queries(w, step=i)).cuda() for i in range(8)]
    out = torch.empty_like(qs[0])
    ws = insts[0].workspace(Hq)
    stream = torch.cuda.current_stream().cuda_stream
    lib = hkv._lib
    used = [0] * R

    def step(i):
        r = i % R
        c, u = insts[r], used[r]
        st = lib.hkv_append_decode(c.handle, ctypes.byref(c.desc), newk[u].data_ptr(), newv[u].data_ptr(),
                                   qs[i % 8].data_ptr(), Hq, out.data_ptr(), None, ws.data_ptr(), ws.numel(), stream)
        if st:
            raise hkv.HKVError(st, "ragged step")
        used[r] += 1
        return sum(decode_bytes(n + used[r], H, Hq, d) + append_bytes(1, H, d) for n in lens0)

    for i in range(warmup):
        step(i)
    res = timed_trials(torch, step, warmup, steps, trials)
    nbytes = statistics.mean(res.pop("rets"))
    last = res["next"] - 1
    r_last = last % R
    got = out.cpu().numpy()
    chk = torch.empty_like(out)
    insts[r_last].decode(qs[last % 8], out=chk, workspace=ws)
    torch.cuda.synchronize()
    record_check(out_close(got, chk.cpu().numpy(), "ragged: last timed output vs hkv_decode_attn recompute"))
    import oracle.hkv_oracle as orc
    b0 = int(np.argmax(lens0))
    n_b = lens0[b0] + used[r_last]
    st = orc.build_state(wl.tokens(w, b0, 0, n_b, "k"), wl.tokens(w, b0, 0, n_b, "v"), w.hot_tokens, w.block_size)
    o_ref, _ = orc.decode(qs[last % 8].cpu().numpy()[b0], st)
    record_check(out_close(got[b0], o_ref, f"ragged: last timed output, longest sequence {b0}, vs the fp64 oracle"))
    for c in insts:
        c.close()
    del insts
    torch.cuda.empty_cache()
    return {"workload": f"ragged: {B} sequences, lengths {min(lens0)}..{max(lens0)} (seeded uniform), permuted "
                        f"physical blocks, step = fused append 1 token/seq + dense decode", "steps": steps,
            "ms_per_step": res["ms_per_step"], "trials_ms": res["trials_ms"],
            "gbs": nbytes / (res["ms_per_step"] * 1e-3) / 1e9,
            "pct_hbm_peak": 100 * nbytes / (res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_step": nbytes,
            "roofline": roofline("decode_kernel_ordered (fused append + decode, batch plan)", nbytes,
                                 res["device_ms_per_step"], "ragged")}


def leg_graph(hkv, torch, args, steps=640, R=64):
    """The llama8b step replayed from a HIP graph (captured once: one fused launch per instance) against
    the same launches issued one by one."""
    import workloads as wl
    w = wl.WORKLOADS["llama8b"]
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    n0 = w.context - 1
    reps = -(-steps // R)
    cap = n0 + 2 * reps + 8
    insts = [hkv.HybridKVCache(H, d, B, cap) for _ in range(R)]
    kh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), 0, n0, "k")).cuda()
    vh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), 0, n0, "v")).cuda()
    for c in insts:
        c.append(kh, vh)
    del kh, vh
    newk = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, 1, "k")).cuda()
    newv = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, 1, "v")).cuda()
    q = torch.from_numpy(wl.queries(w)).cuda()
    out = torch.empty_like(q)
    ws = insts[0].workspace(Hq)
    lib = hkv._lib
    torch.cuda.synchronize()

    def all_instances(stream):
        for c in insts:
            st = lib.hkv_append_decode(c.handle, ctypes.byref(c.desc), newk.data_ptr(), newv.data_ptr(), q.data_ptr(),
                                       Hq, out.data_ptr(), None, ws.data_ptr(), ws.numel(), stream)
            if st:
                raise hkv.HKVError(st, "hkv_append_decode")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        all_instances(side.cuda_stream)  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        all_instances(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    ms_graph = (time.perf_counter() - t0) * 1e3 / (reps * R)
    stream = torch.cuda.current_stream().cuda_stream
    t0 = time.perf_counter()
    for _ in range(reps - 1):
        all_instances(stream)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / ((reps - 1) * R)
    for c in insts:
        c.close()
    del insts
    torch.cuda.empty_cache()
    step_b = B * (decode_bytes(n0 + 2, H, Hq, d) + append_bytes(1, H, d))
    return {"what": "llama8b step: one graph of 64 fused launches (one per instance) replayed, vs the same launches "
                    "issued eagerly", "ms_per_step_graph": ms_graph, "ms_per_step_eager": ms_eager,
            "gbs_graph": step_b / (ms_graph * 1e-3) / 1e9, "steps": reps * R}


def phase_breakdown(hkv, torch, w, n0, R=64, rounds=3):
    """Per-workgroup phase timestamps (hkv_phase_stamps) of one fused step launch among back-to-back
    launches over R rotating instances: per role (cold split; the append workgroup, which attends the
    hot window and then appends and attends the tail block), when its work was done, and the append
    workgroup's phases; when the merges were done.  Times in us from the first workgroup's start
    (100 MHz clock)."""
    import workloads as wl
    B, H, Hq, d = w.batch, w.n_kv_heads, w.n_q_heads, w.head_dim
    insts = [Inst(hkv, w, n0 + rounds + 2) for _ in range(R)]
    for s0 in range(0, n0, 16384):
        cnt = min(16384, n0 - s0)
        kh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s0, cnt, "k")).cuda()
        vh = torch.from_numpy(wl.batch_tokens(w, list(range(B)), s0, cnt, "v")).cuda()
        for it in insts:
            it.c.append(kh, vh)
    kn = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, rounds, "k")).cuda()
    vn = torch.from_numpy(wl.batch_tokens(w, list(range(B)), n0, rounds, "v")).cuda()
    q = torch.from_numpy(wl.queries(w)).cuda()
    out = torch.empty_like(q)
    ws = insts[0].c.workspace(Hq)
    buf = torch.zeros(B * H * 160 * 8, dtype=torch.int64, device="cuda")
    for r in range(rounds):
        for i, it in enumerate(insts):
            mark = r == rounds - 1 and i == R // 2
            if mark:
                hkv.hkv_phase_stamps(it.c.handle, buf)
            it.c.append_decode(kn[:, r].contiguous(), vn[:, r].contiguous(), q, out=out, workspace=ws)
            if mark:
                hkv.hkv_phase_stamps(it.c.handle, None)
    torch.cuda.synchronize()
    flat = buf.cpu().numpy()
    for it in insts:
        it.c.close()
    del insts
    torch.cuda.empty_cache()
    rows = flat.reshape(-1, 8)
    nparts = int((rows[:, 0] != 0).sum()) // (B * H)
    a = rows[:B * H * nparts].reshape(B * H, nparts, 8).astype(np.int64)
    t0 = a[:, :, 0].min()
    us = lambda v: (np.asarray(v, np.float64) - t0) / 100.0
    pct = lambda v: {f"p{p}": round(float(np.percentile(v, p)), 2) for p in (0, 50, 100)}
    cold, app = a[:, :nparts - 1], a[:, nparts - 1]
    merged = a[:, :, 3].max(axis=1)
    last = a[:, :, 1].max(axis=1)
    return {"context": n0 + rounds, "batch": B, "workgroups_per_pair": int(nparts),
            "cold_split_done_us": pct(us(cold[:, :, 1])), "append_done_us": pct(us(app[:, 1])),
            "append_phases_us": {"loads_and_hot_window": pct((app[:, 4] - app[:, 0]) / 100.0),
                                 "coding": pct((app[:, 5] - app[:, 4]) / 100.0),
                                 "code_stores": pct((app[:, 6] - app[:, 5]) / 100.0),
                                 "block_attention": pct((app[:, 7] - app[:, 6]) / 100.0),
                                 "partial_and_arrival": pct((app[:, 1] - app[:, 7]) / 100.0)},
            "merge_done_us": pct(us(merged)), "merge_after_last_arrival_us": pct((merged - last) / 100.0),
            "last_to_arrive": {"cold": int((np.argmax(a[:, :, 1], axis=1) < nparts - 1).sum()),
                               "append": int((np.argmax(a[:, :, 1], axis=1) == nparts - 1).sum())}}


def leg_phases(hkv, torch, args):
    """Phase breakdown of the llama8b fused step (2048 tokens) and of the same step at 544 tokens
    (8 MB: what remains is the step's fixed chain)."""
    import dataclasses
    import workloads as wl
    w = wl.WORKLOADS["llama8b"]
    log("phases: llama8b fused step, per-workgroup timestamps")
    res = {"what": "hkv_phase_stamps of one fused step launch among back-to-back launches (64 instances)",
           "llama8b": phase_breakdown(hkv, torch, w, w.context - 3)}
    res["llama8b_544_tokens"] = phase_breakdown(hkv, torch, dataclasses.replace(w, context=544), 541)
    return res


def leg_read_floor(hkv, torch, args, nbytes=34_406_400, R=64, reps=20):
    """One-launch read of the llama8b step's bytes (34.4 MB, 64 rotating buffers, 16-byte non-temporal
    loads) over launch shapes: the floor a one-launch decode of that size is measured against."""
    bufs = [torch.ones(nbytes // 2, dtype=torch.float16, device="cuda") for _ in range(R)]
    sink = torch.zeros(2048 * 1024, dtype=torch.int32, device="cuda")
    shapes = [(256, 1024), (512, 512), (1024, 256), (2048, 256), (4096, 256)]
    res = []
    for wg, th in shapes:
        def step(i, wg=wg, th=th):
            hkv.hkv_read_probe(bufs[i % R], nbytes, wg, th, sink)
        for i in range(R):
            step(i)
        t = timed_trials(torch, step, 0, R * reps, args.trials)
        ms = t["device_ms_per_step"]
        res.append({"workgroups": wg, "threads": th, "device_ms_per_launch": round(ms, 6),
                    "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    del bufs
    torch.cuda.empty_cache()
    best = min(res, key=lambda x: x["device_ms_per_launch"])
    return {"what": "hkv_read_probe: one launch reading 34.4 MB once (the llama8b step's algorithmic bytes), "
                    "64 rotating buffers", "bytes": nbytes, "shapes": res, "best": best}


def leg_prefill(hkv, torch, args):
    """Bulk append (a prompt's whole K/V in one hkv_append call into an empty cache): the
    quantise launch (every touched block coded from FP16) and the ring/tail launch.  Two shapes:
    the llama8b layer's 8 sequences x 2048 tokens, and the 32768-token top-K workload's fill chunk,
    16 sequences x 8192 tokens.  Each trial empties R instances (seq_len 0, outside the timed
    region) and appends the same tokens to each, back to back."""
    import oracle.hkv_oracle as orc
    import workloads as wl
    out = {"what": "hkv_append of a whole prompt into empty caches (append_quant_kernel + append_ring_kernel)"}
    for name, wname, n, R in (("llama8b_2048", "llama8b", 2048, 16), ("topk_8192", "topk", 8192, 4)):
        w = wl.WORKLOADS[wname]
        B, H, d, T, S = w.batch, w.n_kv_heads, w.head_dim, w.hot_tokens, w.block_size
        log(f"prefill {name}: {R} instances of B={B}, {n} tokens per sequence")
        insts = [hkv.HybridKVCache(H, d, B, n) for _ in range(R)]
        kb = torch.from_numpy(wl.batch_tokens(w, list(range(B)), 0, n, "k")).cuda()
        vb = torch.from_numpy(wl.batch_tokens(w, list(range(B)), 0, n, "v")).cuda()

        def reset():
            for c in insts:
                c.seq_len.zero_()
                c.seq_len_host[:] = 0
            torch.cuda.synchronize()

        host, dev = [], []
        for _ in range(1 + args.trials):  # the first round warms up
            reset()
            t0 = time.perf_counter()
            for c in insts:
                c.append(kb, vb)
            torch.cuda.synchronize()
            host.append((time.perf_counter() - t0) * 1e3 / R)
            reset()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for c in insts:
                c.append(kb, vb)
            e1.record()
            torch.cuda.synchronize()
            dev.append(e0.elapsed_time(e1) / R)
        host, dev = host[1:], dev[1:]
        n_cold = n - T
        blocks = -(-n_cold // S)
        tile = S * d  # bytes of one 8-bit (block, kv-head, K|V) tile
        nbytes = (B * n * H * d * 2 * 2            # every new K and V row read (fp16)
                  + B * blocks * H * 2 * tile      # the touched tiles written
                  + B * blocks * H * 2 * 4         # their scales
                  + B * (n_cold % S) * H * d * 2 * 2  # the partial block's rows into the tail shadow
                  + B * T * H * d * 2 * 2)         # the hot ring
        ms = statistics.median(dev)
        # the last trial's caches: all instances equal, and sequence 0's codes and scales equal the oracle's
        # (sequence 0's logical blocks are physical blocks 0, 1, ... in the default placement)
        c0 = insts[0]
        same = all(torch.equal(c0.cold, c.cold) and torch.equal(c0.scales, c.scales) and torch.equal(c0.hot, c.hot)
                   for c in insts[1:])
        record_check({"what": f"prefill {name}: every instance holds the same bytes", "ok": bool(same)})
        st = orc.build_state(kb[0].cpu().numpy(), vb[0].cpu().numpy(), T, S)
        codes = c0.cold_codes()
        scales = c0.scale_array()
        nb = min(4, blocks)
        ok = bool(np.array_equal(codes[:nb], st.codes[:nb]) and np.array_equal(scales[:nb], st.scales[:nb]))
        record_check({"what": f"prefill {name}: sequence 0, blocks 0-{nb - 1}: codes and scales vs the fp64 oracle "
                              "(bitwise)", "ok": ok})
        out[name] = {"batch": B, "tokens": n, "instances": R, "ms_per_call": round(statistics.median(host), 6),
                     "trials_ms": [round(x, 6) for x in host],
                     "roofline": roofline("append_quant_kernel + append_ring_kernel (one hkv_append call)", nbytes, ms,
                                          f"prefill_{name}")}
        del insts, kb, vb
        torch.cuda.empty_cache()
    return out


def host_info():
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count()
    return {"cpu_count": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model, "blas_threads": int(blas)}


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on the same step (append one token + decode), 8 sequences, bounded time."""
    import oracle.hkv_oracle as orc
    import workloads as wl
    info = host_info()
    n0 = w.context - 1
    S, T = w.block_size, w.hot_tokens
    H, Hq, d = w.n_kv_heads, w.n_q_heads, w.head_dim
    extra = 512  # appended tokens the sample may use (bounds the sample as well as the time budget)
    hist_k = [wl.tokens(w, b, 0, n0 + extra, "k") for b in range(w.batch)]
    hist_v = [wl.tokens(w, b, 0, n0 + extra, "v") for b in range(w.batch)]
    states = [orc.build_state(hist_k[b][:n0], hist_v[b][:n0], T, S) for b in range(w.batch)]
    steps = 0
    nbytes = 0
    t0 = time.perf_counter()
    while True:
        for b in range(w.batch):
            st = states[b]
            n1 = st.n_tokens + 1
            n_hot, n_cold = orc.split_history(n1, T)
            j = (n_cold - 1) // S
            kr, vr = hist_k[b][j * S:n_cold], hist_v[b][j * S:n_cold]
            codes, scales = orc.quantize_block(kr, vr, S)
            if j >= st.n_blocks:
                st.codes = np.concatenate([st.codes, codes[None]])
                st.scales = np.concatenate([st.scales, scales[None]])
                st.n_valid = np.concatenate([st.n_valid, [n_cold - j * S]])
            else:
                st.codes[j], st.scales[j], st.n_valid[j] = codes, scales, n_cold - j * S
            st.hot_k, st.hot_v = hist_k[b][n_cold:n1], hist_v[b][n_cold:n1]
            st.n_tokens = n1
            orc.decode(wl.query(w, b, steps), st)
            nbytes += decode_bytes(n1, H, Hq, d) + append_bytes(1, H, d)
        steps += 1
        if time.perf_counter() - t0 >= budget_s or steps >= extra:
            break
    el = time.perf_counter() - t0
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"{steps} steps x {w.batch} sequences of the llama8b step (fp64 NumPy oracle: re-quantise "
                      f"the touched block + dense decode), {el:.1f} s; cores = the BLAS threads of its matrix-vector "
                      f"products (the rest of the oracle runs on one thread)",
            "ms_per_step": el * 1e3 / steps, "host": info}


def copy_calibration(torch, mib=256, reps=4):
    """A plain elementwise copy of a known size (reads and writes `mib` MiB per launch).  Hardware
    counters of this launch calibrate the FETCH_SIZE / WRITE_SIZE readings of the path's kernels."""
    x = torch.ones(mib << 19, dtype=torch.float16, device="cuda")
    y = torch.empty_like(x)
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    return {"kernel": "torch.neg (elementwise fp16)", "bytes_read": mib << 20, "bytes_written": mib << 20,
            "launches": reps}


LEGS = ("llama8b", "separate", "long", "llama8b_int4", "long_int4", "llama8b_fp16", "long_fp16", "sparse", "ragged", "phases",
        "graph", "read_floor", "prefill", "cpu")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--instances", type=int, default=64)
    ap.add_argument("--leg", default="all", help=f"comma-separated subset of {','.join(LEGS)} (default all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a known-size copy kernel (for hardware-counter traffic calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the decode path is built and "
              f"measured on a single MI355X; how it would shard across GPUs is a design note, not a built path)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    legs = LEGS if args.leg == "all" else tuple(x for x in args.leg.split(",") if x)
    for x in legs:
        if x not in LEGS:
            ap.error(f"unknown leg {x}")
    if args.no_cpu_baseline:
        legs = tuple(x for x in legs if x != "cpu")
    import torch
    import int8_kv_cache_hkv_amd as hkv
    import workloads as wl
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = wl.WORKLOADS["llama8b"]
    H, Hq, d = w.n_kv_heads, w.n_q_heads, w.head_dim
    res = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": "llama8b: Llama-3-8B-shaped layer, batch 8, 32 q / 8 kv heads, head_dim 128, "
                                  "2048 cached tokens (32 FP16 hot + 31 full + 1 half INT8 block), step = append 1 "
                                  "token/seq + dense decode (one fused launch)",
                      "batch": w.batch, "context": w.context, "hot_tokens": w.hot_tokens,
                      "block_size": w.block_size, "quant_bits": w.quant_bits, "instances": args.instances},
           "arithmetic": "int8 codes and fp16 values as exact fp16 MFMA operands, fp32 accumulation and softmax",
           "trials": args.trials}
    if "llama8b" in legs:
        _, r = leg_llama8b(hkv, torch, args)
        gbs, ms = r["gbs"], r["ms_per_step"]
        res.update({
            "value": round(gbs, 2), "ms_per_step": round(ms, 6), "trials_ms": r["trials_ms"],
            "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "queries_per_s": round(w.batch / (ms * 1e-3), 1),
            "head_queries_per_s": round(w.batch * Hq / (ms * 1e-3), 1),
            "bytes_per_step": int(r["bytes_per_step"]),
            "roofline": roofline("decode_kernel (fused append + decode)", r["kernel_bytes_per_step"],
                                 r["device_ms_per_step"], "llama8b"),
        })
    if "separate" in legs:
        res["separate_calls"] = leg_separate(hkv, torch, args)
    if "long" in legs:
        res["long"] = leg_long(hkv, torch, args)
    for name in ("llama8b", "long"):
        for bits, tag in ((4, "int4"), (0, "fp16")):
            if f"{name}_{tag}" in legs:
                res[f"{name}_{tag}"] = leg_width(hkv, torch, args, name, bits)
    if "sparse" in legs:
        res["sparse"] = leg_sparse(hkv, torch, args)
    if "ragged" in legs:
        res["ragged"] = leg_ragged(hkv, torch, args)
    if "graph" in legs:
        res["hip_graph"] = leg_graph(hkv, torch, args)
    if "phases" in legs:
        res["phases"] = leg_phases(hkv, torch, args)
    if "read_floor" in legs:
        res["read_floor"] = leg_read_floor(hkv, torch, args)
    if "prefill" in legs:
        res["prefill"] = leg_prefill(hkv, torch, args)
    if args.copy_calibration:
        res["copy_calibration"] = copy_calibration(torch)
    if "cpu" in legs:
        log("cpu baseline (fp64 oracle)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    res["self_check"] = {"passed": all(c["ok"] for c in CHECKS), "checks": CHECKS}
    print(json.dumps(res), flush=True)
    if not res["self_check"]["passed"]:
        sys.exit(3)


if __name__ == "__main__":
    main()
