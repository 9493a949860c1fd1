"""GPU: the split-K decomposition does not change the result beyond fp32 rounding.

A decode's cold blocks are cut into splits whose partial (m, l, acc) records are merged by their
log-sum-exp (Hybrid KV Cache page, 2.3: split-K over the cold blocks, then an LSE combine of the
partial softmax states).  The launch plan is forced through the plan override: static plans of 1
to 128 splits, and claim plans on grids of several sizes.  Each output is checked against the fp64
oracle, and the outputs of different plans against each other: lse within 2e-5, the fp16 output
within one fp16 rounding step plus fp32 reassociation.  A static plan takes no claims, so two calls
under it agree bit for bit.
"""
import dataclasses

import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

LSE_SPLIT_ABS = 2e-5
OUT_SPLIT_ABS = 1.5e-3   # one fp16 step at |out| < 2 is 9.8e-4, plus fp32 reassociation


def _decode(cache, q_np):
    torch = gh.torch_mod()
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cache.decode(q, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _states(w, lens):
    res = []
    for b, n in enumerate(lens):
        k, v = gh.history(w, b, n)
        res.append(orc.build_state(k, v, w.hot_tokens, w.block_size, w.quant_bits))
    return res


def _across(ref, got, what):
    o0, l0 = ref
    o1, l1 = got
    dl = float(np.max(np.abs(l1 - l0)))
    do = float(np.max(np.abs(o1.astype(np.float32) - o0.astype(np.float32))))
    gh.log(f"  {what}: max |d lse| {dl:.2e}, max |d out| {do:.2e} against one split")
    assert dl <= LSE_SPLIT_ABS, f"{what}: lse moved by {dl}"
    assert do <= OUT_SPLIT_ABS, f"{what}: output moved by {do}"


@pytest.mark.parametrize("bits", [8, 4, 0])
def test_static_split_counts(bits):
    """98 cold units (97 full blocks and a partial one) under static plans of 1, 2, 3, 5, 8, 25 and
    128 (= 25: four units per split at least) splits."""
    import int8_kv_cache_hkv_amd as hkv
    w = dataclasses.replace(wl.WORKLOADS["llama8b"], name=f"splits{bits}", batch=4, quant_bits=bits)
    n = 32 + 64 * 97 + 11
    cache = gh.make_cache(w, n + 8)
    gh.fill(cache, w, [n] * w.batch)
    st = _states(w, [n] * w.batch)
    q = wl.queries(w)[:w.batch]
    refs = [orc.decode(q[b], st[b]) for b in range(w.batch)]
    base = None
    for ns in [1, 2, 3, 5, 8, 25, 128]:
        hkv.hkv_plan_override(cache.handle, ns, 0)
        got = _decode(cache, q)
        again = _decode(cache, q)
        assert np.array_equal(got[0].view(np.uint16), again[0].view(np.uint16)) and \
            np.array_equal(got[1], again[1]), f"{ns} splits: two calls differ"
        for b in range(w.batch):
            gh.compare_out(got[0][b], refs[b][0], f"{bits}-bit {ns} splits b={b}")
            gh.compare_lse(got[1][b], refs[b][1], f"{bits}-bit {ns} splits b={b}")
        if base is None:
            base = got
        else:
            _across(base, got, f"{bits}-bit {ns} splits")
    hkv.hkv_plan_override(cache.handle, 0, 0)
    auto = _decode(cache, q)
    _across(base, auto, f"{bits}-bit automatic plan")
    cache.close()


def test_claim_grids_and_fused_step():
    """A resident claim plan (about 2000 cold units per (sequence, kv-head)) on claim grids of 3, 64,
    256, 512, 1024 and 2048 workgroups, and the fused append + decode step under static and claim
    plans: every output against the oracle and against the one-split plan."""
    import int8_kv_cache_hkv_amd as hkv
    w = dataclasses.replace(wl.WORKLOADS["long"], name="split_claims", batch=2, n_kv_heads=4, n_q_heads=16)
    n = 32 + 64 * 2000 + 40
    cache = gh.make_cache(w, n + 8)
    gh.fill(cache, w, [n] * w.batch, chunk=8192)
    st = _states(w, [n] * w.batch)
    q = wl.queries(w)[:w.batch]
    refs = [orc.decode(q[b], st[b]) for b in range(w.batch)]
    hkv.hkv_plan_override(cache.handle, 1, 0)
    base = _decode(cache, q)
    for b in range(w.batch):
        gh.compare_out(base[0][b], refs[b][0], f"one split b={b}")
        gh.compare_lse(base[1][b], refs[b][1], f"one split b={b}")
    for grid in [3, 64, 256, 512, 1024, 2048]:
        hkv.hkv_plan_override(cache.handle, 0, grid)
        got = _decode(cache, q)
        for b in range(w.batch):
            gh.compare_out(got[0][b], refs[b][0], f"claim grid {grid} b={b}")
        _across(base, got, f"claim grid {grid}")
    # fused step: append token n of each sequence, decode over n + 1 tokens
    torch = gh.torch_mod()
    st1 = _states(w, [n + 1] * w.batch)
    refs1 = [orc.decode(q[b], st1[b]) for b in range(w.batch)]
    kb = np.stack([wl.tokens(w, b, n, 1, "k")[0] for b in range(w.batch)])
    vb = np.stack([wl.tokens(w, b, n, 1, "v")[0] for b in range(w.batch)])
    outs = []
    for ns, grid in [(1, 0), (7, 0), (0, 384)]:
        c2 = gh.make_cache(w, n + 8)
        gh.fill(c2, w, [n] * w.batch, chunk=8192)
        hkv.hkv_plan_override(c2.handle, ns, grid)
        qt = gh.upload(q)
        out = torch.empty_like(qt)
        lse = torch.empty(qt.shape[:2], dtype=torch.float32, device=qt.device)
        c2.append_decode(gh.upload(kb), gh.upload(vb), qt, out=out, lse=lse)
        torch.cuda.synchronize()
        got = (out.cpu().numpy(), lse.cpu().numpy())
        for b in range(w.batch):
            gh.compare_out(got[0][b], refs1[b][0], f"fused splits={ns} grid={grid} b={b}")
            gh.compare_lse(got[1][b], refs1[b][1], f"fused splits={ns} grid={grid} b={b}")
        outs.append(got)
        c2.close()
    for got, tag in zip(outs[1:], ["7 splits", "claim grid 384"]):
        _across(outs[0], got, f"fused {tag}")
    cache.close()

