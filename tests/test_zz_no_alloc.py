"""GPU: hkv_decode_attn_noalloc (no workspace argument, fixed device scratch) against
hkv_decode_attn on the same caches, through the C ABI: consecutive calls with a larger then a
smaller input, a plan whose waves claim blocks from counters in the scratch (the counters must be
back at zero for the next call), and a sparse call; each output and lse against the workspace
entry point's to the parity bar, and against the fp64 oracle."""
import ctypes

import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


def _both(cache, q_np, sel=None, k_sel=0):
    """(out, lse) of hkv_decode_attn with a workspace and of hkv_decode_attn_noalloc."""
    import int8_kv_cache_hkv_amd as hkv
    torch = gh.torch_mod()
    q = gh.upload(q_np)
    res = []
    for noalloc in (False, True):
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device=q.device)
        if noalloc:
            hkv.hkv_decode_attn_noalloc(cache.handle, cache.desc, q, out, lse=lse, sel_idx=sel, k_sel=k_sel)
        else:
            cache.decode(q, out=out, lse=lse, sel_idx=sel, k_sel=k_sel)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


def _check(cache, w, lens, q, what, sel=None, k_sel=0):
    (o_ws, l_ws), (o_na, l_na) = _both(cache, q, sel, k_sel)
    gh.compare_out(o_na.astype(np.float64), o_ws.astype(np.float64), f"{what}: noalloc vs workspace")
    gh.compare_lse(l_na, l_ws.astype(np.float64), f"{what}: noalloc vs workspace")
    for b in range(len(lens)):
        st = orc.build_state(*gh.history(w, b, lens[b]), w.hot_tokens, w.block_size)
        if sel is None:
            o_ref, l_ref = orc.decode(q[b], st)
        else:
            o_ref, l_ref = orc.sparse_decode(q[b], st, sel.cpu().numpy()[b])
        gh.compare_out(o_na[b], o_ref, f"{what}: noalloc b={b}")
        gh.compare_lse(l_na[b], l_ref, f"{what}: noalloc b={b}")


def test_noalloc_matches_workspace_entry_point():
    import dataclasses
    torch = gh.torch_mod()
    # call 1: 4 sequences x 8 kv-heads of 700 cold blocks: splits of >= 16 blocks claim them from the
    # counters in the scratch
    w1 = dataclasses.replace(wl.WORKLOADS["llama8b"], name="noalloc_big", batch=4)
    lens1 = [32 + 64 * 700 + 9, 32 + 64 * 650, 32 + 64 * 699 + 63, 32 + 64 * 300 + 1]
    big = gh.make_cache(w1, max(lens1) + 8)
    gh.fill(big, w1, lens1, chunk=8192)
    q1 = wl.queries(w1, step=4)
    _check(big, w1, lens1, q1, "claim plan")
    # call 2: a smaller input (2 sequences of the tiny shape)
    w2 = dataclasses.replace(wl.WORKLOADS["tiny"], name="noalloc_small", batch=2)
    lens2 = [288, 97]
    small = gh.make_cache(w2, 400)
    gh.fill(small, w2, lens2)
    q2 = wl.queries(w2, step=2)
    _check(small, w2, lens2, q2, "small dense")
    # call 3: sparse, on the small cache
    rng = np.random.default_rng(3)
    st = [orc.build_state(*gh.history(w2, b, n), 32, 64) for b, n in enumerate(lens2)]
    k_sel = 40
    sel = np.stack([rng.integers(0, s.n_cold, size=(w2.n_kv_heads, k_sel)) for s in st]).astype(np.int32)
    _check(small, w2, lens2, q2, "small sparse", sel=gh.upload(sel), k_sel=k_sel)
    # call 4: the claim plan again (its counters were reset by the first call)
    _check(big, w1, lens1, wl.queries(w1, step=5), "claim plan again")
    big.close()
    small.close()


def test_noalloc_rejects_oversized_scratch():
    """A call needing more than the fixed 32 MiB of scratch returns HKV_ERR_WORKSPACE before any
    launch (top-K-sized workspaces are larger, but a decode's partials for 4096 sequences x 8 kv-heads
    of up to 128 splits are too)."""
    import int8_kv_cache_hkv_amd as hkv
    h = hkv.hkv_create(8, 128)
    try:
        B = 4096
        lens = np.full(B, 32 + 64 * 8192, dtype=np.int32)
        base = 1 << 40
        desc = hkv.CacheDesc(B, 8192, B * 8192, base, base + 4096, base + 8192, base + 12288, base + 16384,
                             base + 20480, lens.ctypes.data)
        need = hkv.hkv_workspace_bytes(h, desc, 32)
        assert need > (32 << 20)
        q = 1 << 41
        st = hkv._lib.hkv_decode_attn_noalloc(h, ctypes.byref(desc), q, 32, None, 0, q, None, None)
        assert st == -5
    finally:
        hkv.hkv_destroy(h)
