"""GPU parity of the compacted sparse store against the fp64 oracle, through the C ABI.

KV Cache reuse page 2 (Index-Aware Cache Layout: the selected tokens' KV re-packed into a compact
block, the only part loaded) and 2.1 (aligned, padded blocks).  The store's counts, rows (codes or
fp16 values) and per-token scales are compared bit for bit with the oracle's store of the same
selection; the decode over hot zone + store against the oracle within max |d| 4e-3 / mean |d| 5e-4
(lse 1e-3), for the three cold widths, every (head_dim, group) instance, selection widths that are
not multiples of 64, masked / out-of-range / duplicate entries, and the 32768-token top-K workload.
"""
import dataclasses

import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh
from tests import oracle_jobs as oj

pytestmark = pytest.mark.gpu


def _w(name, bits, **kw):
    return dataclasses.replace(wl.WORKLOADS[name], name=f"{name}_st{bits}", quant_bits=bits, **kw)


def _check_store(cache, store, k_sel, states, sels):
    counts, k_rows, v_rows, scales = cache.store_rows(store, k_sel)
    for b, (st, sel) in enumerate(zip(states, sels)):
        want = orc.sparse_store(st, sel)
        assert counts[b].tolist() == want.counts.tolist(), (b, counts[b], want.counts)
        for h in range(cache.H):
            m = int(want.counts[h])
            for got, ref in ((k_rows[b, h, :m], want.k_codes[h]), (v_rows[b, h, :m], want.v_codes[h])):
                ref = np.asarray(ref)
                if got.dtype == np.float16:
                    got, ref = got.view(np.uint16), ref.astype(np.float16).view(np.uint16)
                assert np.array_equal(got, ref), (b, h)
            assert np.array_equal(scales[b, h, :m, 0].view(np.uint32), want.k_scales[h].view(np.uint32))
            assert np.array_equal(scales[b, h, :m, 1].view(np.uint32), want.v_scales[h].view(np.uint32))


def _decode_store(cache, q_np, store, k_sel):
    torch = gh.torch_mod()
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cache.decode_store(q, store, k_sel, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("bits", [8, 4, 0])
@pytest.mark.parametrize("k_sel", [1, 37, 64, 100, 512])
def test_store_explicit_selections(bits, k_sel):
    """Caller-built selections with -1, out-of-range and duplicate entries: store bytes bit-exact, decode
    over it equal to the oracle's sparse decode."""
    torch = gh.torch_mod()
    w = _w("tiny", bits, batch=2)
    lens = [32 + 64 * 12 + 9, 32 + 64 * 3 + 1]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    states = [orc.build_state(*gh.history(w, b, n), 32, 64, bits) for b, n in enumerate(lens)]
    rng = np.random.default_rng(1000 + k_sel + bits)
    sel = np.stack([rng.integers(0, s.n_cold, size=(w.n_kv_heads, k_sel)) for s in states]).astype(np.int32)
    m = rng.random(sel.shape)
    sel[m < 0.1] = -1
    sel[(m >= 0.1) & (m < 0.14)] = 10 ** 6
    store = cache.sparse_store(gh.upload(sel), k_sel)
    torch.cuda.synchronize()
    _check_store(cache, store, k_sel, states, sel)
    q = wl.queries(w, step=5)
    out, lse = _decode_store(cache, q, store, k_sel)
    for b, st in enumerate(states):
        clean = np.where((sel[b] >= 0) & (sel[b] < st.n_cold), sel[b], -1)
        o_ref, l_ref = orc.sparse_decode(q[b], st, clean)
        gh.compare_out(out[b], o_ref, f"{bits}-bit k={k_sel} store b={b}")
        gh.compare_lse(lse[b], l_ref, f"{bits}-bit k={k_sel} store b={b}")
    cache.close()


@pytest.mark.parametrize("d,g", [(64, 1), (64, 8), (128, 1), (128, 2), (128, 4), (128, 8)])
def test_store_group_sizes(d, g):
    """Every (head_dim, group) instance of the store decode, on a top-K selection."""
    w = _w("tiny", 8, batch=2, n_q_heads=2 * g, head_dim=d)
    lens = [32 + 64 * 9 + 17, 32 + 64 * 5 + 40]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=9)
    k_sel = 100
    idx = cache.topk(gh.upload(q), k_sel)
    store = cache.sparse_store(idx, k_sel)
    out, lse = _decode_store(cache, q, store, k_sel)
    got = idx.cpu().numpy()
    for b, n in enumerate(lens):
        st = orc.build_state(*gh.history(w, b, n), 32, 64)
        o_ref, l_ref = orc.sparse_decode(q[b], st, got[b])
        gh.compare_out(out[b], o_ref, f"store d={d} g={g} b={b}")
        gh.compare_lse(lse[b], l_ref, f"store d={d} g={g} b={b}")
    cache.close()


@pytest.mark.parametrize("bits", [8, 4])
def test_store_topk_config(bits):
    """The 32768-token top-K workload: selection, store and store decode for all 16 sequences against the
    oracle's sparse decode over the GPU's selection; the store decode equals the gather decode."""
    torch = gh.torch_mod()
    w = _w("topk", bits)
    n, B, k = w.context, w.batch, w.k_sel
    cache = gh.make_cache(w, n)
    gh.fill(cache, w, [n] * B, chunk=8192)
    q = wl.queries(w)
    qd = gh.upload(q)
    idx = cache.topk(qd, k)
    store = cache.sparse_store(idx, k)
    out, lse = _decode_store(cache, q, store, k)
    out_g = torch.empty_like(qd)
    cache.decode(qd, out=out_g, sel_idx=idx, k_sel=k)
    torch.cuda.synchronize()
    gh.compare_out(out.astype(np.float64), out_g.cpu().numpy().astype(np.float64), f"{bits}-bit store vs gather")
    got = idx.cpu().numpy()
    with oj.pool(B) as ex:
        futs = [ex.submit(oj.topk_job, "topk", b, q[b], k, got[b], {"quant_bits": bits}) for b in range(B)]
        for b, f in enumerate(futs):
            _, _, _, _, o_ref, l_ref = f.result()
            gh.compare_out(out[b], o_ref, f"{bits}-bit topk store b={b}")
            gh.compare_lse(lse[b], l_ref, f"{bits}-bit topk store b={b}")
    cache.close()
