"""GPU parity of the 4-bit cold blocks and the FP16 cold zone against the fp64 oracle, through the C ABI.

Hybrid KV Cache page 3.1: quantization_bits is 4 or 8 (INT4 for L2 cold blocks); 5.2:
quantization_bits 0 keeps the cold zone in FP16.  For each width the same bars as the 8-bit path:
codes (or fp16 values), scales, headers, hot ring and lengths bit-exact; fp16 attention output within
max |d| 4e-3 / mean |d| 5e-4 of the fp64 oracle; lse within 1e-3; top-K sets equal outside near-ties.
Cases: the tiny config and ragged lengths, append chunking invariance, the Llama-3-8B-shaped layer
with a fused step, fused steps around block and hot-zone boundaries, every (head_dim, group)
instance (dense, sparse, fused), claim-walk and batch plans, other hot-zone sizes, top-K and sparse
decode, ragged fused steps and (4 bits) the 131072-token workload.
"""
import dataclasses

import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh
from tests import oracle_jobs as oj

pytestmark = pytest.mark.gpu

WIDTHS = [4, 0]


def _w(name, bits, **kw):
    return dataclasses.replace(wl.WORKLOADS[name], name=f"{name}_b{bits}", quant_bits=bits, **kw)


def _states(w, lens, seqs=None):
    seqs = list(range(len(lens))) if seqs is None else seqs
    return [orc.build_state(*gh.history(w, b, n), w.hot_tokens, w.block_size, w.quant_bits)
            for b, n in zip(seqs, lens)]


def _decode(cache, q_np, sel=None, k_sel=0):
    torch = gh.torch_mod()
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cache.decode(q, out=out, lse=lse, sel_idx=sel, k_sel=k_sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _fused(cache, w, cur, q_np):
    torch = gh.torch_mod()
    kb = np.stack([wl.tokens(w, b, cur[b], 1, "k")[0] for b in range(len(cur))])
    vb = np.stack([wl.tokens(w, b, cur[b], 1, "v")[0] for b in range(len(cur))])
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cache.append_decode(gh.upload(kb), gh.upload(vb), q, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _compare(out, lse, q, states, what, seqs=None):
    seqs = list(range(len(states))) if seqs is None else seqs
    for b, st in zip(seqs, states):
        o_ref, l_ref = orc.decode(q[b], st)
        gh.compare_out(out[b], o_ref, f"{what} b={b}")
        gh.compare_lse(lse[b], l_ref, f"{what} b={b}")


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_tiny_and_ragged_lengths(bits):
    """The tiny config and lengths with empty, partial and exact-boundary cold zones."""
    w = _w("tiny", bits)
    for n in (1, 31, 33, 95, 97, 161, 288, 300):
        cache = gh.make_cache(w, 400)
        gh.fill(cache, w, [n])
        st = _states(w, [n])
        gh.check_state(cache, st)
        q = wl.queries(w, step=n)
        out, lse = _decode(cache, q)
        _compare(out, lse, q, st, f"{bits}-bit n={n}")
        cache.close()


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_append_chunking_invariance(bits):
    """A bulk append, single-token appends and random chunks leave identical bytes and outputs."""
    torch = gh.torch_mod()
    w = _w("tiny", bits)
    n = 350
    rng = np.random.default_rng(5)
    caches = []
    for mode in ("bulk", "single", "random"):
        cache = gh.make_cache(w, 400)
        if mode == "bulk":
            gh.fill(cache, w, [n])
        elif mode == "single":
            for p in range(n):
                gh.fill(cache, w, [p + 1], start=[p])
        else:
            p = 0
            while p < n:
                step = int(min(n - p, rng.integers(1, 90)))
                gh.fill(cache, w, [p + step], start=[p])
                p += step
        caches.append(cache)
    ref = caches[0]
    for c in caches[1:]:
        assert torch.equal(ref.cold, c.cold) and torch.equal(ref.scales, c.scales)
        assert torch.equal(ref.headers, c.headers) and torch.equal(ref.hot, c.hot)
    q = wl.queries(w, step=7)
    outs = [_decode(c, q)[0] for c in caches]
    assert all(np.array_equal(outs[0].view(np.uint16), o.view(np.uint16)) for o in outs[1:])
    gh.check_state(ref, _states(w, [n]))


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_llama8b(bits):
    """The Llama-3-8B-shaped layer at full size (K outlier channels), a fused step, and the fused
    step's cache bytes equal to those of hkv_append + hkv_decode_attn."""
    w = _w("llama8b", bits)
    n = w.context
    a = gh.make_cache(w, n + 8)
    b = gh.make_cache(w, n + 8)
    gh.fill(a, w, [n - 1] * w.batch)
    gh.fill(b, w, [n - 1] * w.batch)
    st0 = _states(w, [n - 1] * w.batch)
    gh.check_state(a, st0)
    q0 = wl.queries(w)
    out, lse = _decode(a, q0)
    _compare(out, lse, q0, st0, f"{bits}-bit llama8b n={n - 1}")
    q = wl.queries(w, step=1)
    out_f, lse_f = _fused(a, w, [n - 1] * w.batch, q)
    gh.fill(b, w, [n] * w.batch, start=[n - 1] * w.batch)
    out_s, _ = _decode(b, q)
    st1 = _states(w, [n] * w.batch)
    gh.check_state(a, st1)
    gh.check_state(b, st1)
    assert np.array_equal(a.cold.cpu().numpy(), b.cold.cpu().numpy())
    assert np.array_equal(a.tail.cpu().numpy(), b.tail.cpu().numpy())
    _compare(out_f, lse_f, q, st1, f"{bits}-bit llama8b fused")
    for bb in range(w.batch):
        gh.compare_out(out_s[bb], orc.decode(q[bb], st1[bb])[0], f"{bits}-bit llama8b separate b={bb}")


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_fused_small(bits):
    """Fused steps from lengths where the hot zone is not full, where the spilled token opens a block,
    lands inside one (maximum kept or raised) or completes one."""
    w = _w("tiny", bits)
    for n0 in (0, 5, 31, 32, 33, 40, 95, 96, 97, 159, 160, 161, 287, 300):
        cache = gh.make_cache(w, 400)
        gh.fill(cache, w, [n0])
        q = wl.queries(w, step=n0)
        out, lse = _fused(cache, w, [n0], q)
        st = _states(w, [n0 + 1])
        gh.check_state(cache, st)
        _compare(out, lse, q, st, f"{bits}-bit fused n0={n0}")
        cache.close()


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("d,g", [(64, 1), (64, 8), (128, 1), (128, 2), (128, 4), (128, 8)])
def test_formats_group_sizes(bits, d, g):
    """Every built (head_dim, group) instance, plain, sparse and fused."""
    w = _w("tiny", bits, batch=2, n_q_heads=2 * g, head_dim=d)
    lens = [32 + 64 * 3 + 17, 32 + 64 * 6 + 40]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=7)
    st = _states(w, lens)
    out, lse = _decode(cache, q)
    _compare(out, lse, q, st, f"{bits}-bit d={d} g={g} dense")
    k_sel = 50
    rng = np.random.default_rng(10 * d + g)
    sel = np.stack([rng.integers(0, s.n_cold, size=(w.n_kv_heads, k_sel)) for s in st]).astype(np.int32)
    out_s, lse_s = _decode(cache, q, sel=gh.upload(sel), k_sel=k_sel)
    for b in range(2):
        o_ref, l_ref = orc.sparse_decode(q[b], st[b], sel[b])
        gh.compare_out(out_s[b], o_ref, f"{bits}-bit d={d} g={g} sparse b={b}")
        gh.compare_lse(lse_s[b], l_ref, f"{bits}-bit d={d} g={g} sparse b={b}")
    out_f, lse_f = _fused(cache, w, lens, q)
    st1 = _states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    _compare(out_f, lse_f, q, st1, f"{bits}-bit d={d} g={g} fused")


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_claim_walk(bits):
    """32 sequences of 40 tokens to 100 cold blocks at a permuted placement: splits of >= 16 blocks claim
    them from counters; plain decode twice, then a fused step."""
    w = _w("llama8b", bits, batch=32)
    rng = np.random.default_rng(11)
    lens = [40, 32 + 64 * 11, 32 + 64 * 12 + 5, 32 + 64 * 100] + rng.integers(100, 32 + 64 * 100, 28).tolist()
    cap = max(lens) + 8
    mb = -(-(cap - 32) // 64)
    perm = rng.permutation(w.batch * mb).reshape(w.batch, mb)
    cache = gh.make_cache(w, cap, phys_ids=perm)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=7)
    o1, l1 = _decode(cache, q)
    o2, l2 = _decode(cache, q)
    st = _states(w, lens)
    _compare(o1, l1, q, st, f"{bits}-bit claim first")
    _compare(o2, l2, q, st, f"{bits}-bit claim second")
    out_f, lse_f = _fused(cache, w, lens, q)
    _compare(out_f, lse_f, q, _states(w, [n + 1 for n in lens]), f"{bits}-bit claim fused")


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_batch_plan(bits):
    """200 short sequences x 2 kv-heads: a batch plan in the longest-first table order, plain and fused."""
    w = _w("tiny", bits, batch=200)
    rng = np.random.default_rng(200)
    lens = rng.integers(40, 421, 200).tolist()
    cache = gh.make_cache(w, max(lens) + 8)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=5)
    out, lse = _decode(cache, q)
    _compare(out, lse, q, _states(w, lens), f"{bits}-bit batch plan")
    out_f, lse_f = _fused(cache, w, lens, q)
    st1 = _states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    _compare(out_f, lse_f, q, st1, f"{bits}-bit batch plan fused")


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("T", [16, 128])
def test_formats_hot_tokens(bits, T):
    """Other hot-zone sizes: append, dense decode and a fused step; one sequence still all-hot."""
    w = _w("tiny", bits, batch=2, hot_tokens=T)
    lens = [T + 64 * 3 + 17, T - 5]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    st = _states(w, lens)
    gh.check_state(cache, st)
    q = wl.queries(w, step=1)
    out, lse = _decode(cache, q)
    _compare(out, lse, q, st, f"{bits}-bit T={T}")
    out_f, lse_f = _fused(cache, w, lens, q)
    st1 = _states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    _compare(out_f, lse_f, q, st1, f"{bits}-bit T={T} fused")


@pytest.mark.parametrize("bits", WIDTHS)
@pytest.mark.parametrize("n,k", [(32 + 300, 50), (32 + 64 * 9 + 17, 100), (20, 16), (32 + 32768, 512),
                                 (32 + 40007, 300)])
def test_formats_topk_sparse(bits, n, k):
    """Top-K selection (cosine of the 4-bit codes, or of the fp16 keys) and the sparse decode over it."""
    w = _w("tiny", bits)
    cache = gh.make_cache(w, n + 64)
    gh.fill(cache, w, [n])
    st = _states(w, [n])[0]
    q = wl.queries(w, step=3)
    idx = cache.topk(gh.upload(q), k)
    gh.torch_mod().cuda.synchronize()
    got = idx.cpu().numpy()
    want, p, tau = orc.topk_select(q[0], st, k)
    for h in range(w.n_kv_heads):
        gh.compare_topk(got[0, h], want[h], p[h], tau[h], st.n_cold, k, f"{bits}-bit n={n} k={k} h={h}")
    if st.n_cold > 0:
        out, lse = _decode(cache, q, sel=idx, k_sel=k)
        o_ref, l_ref = orc.sparse_decode(q[0], st, got[0])
        gh.compare_out(out[0], o_ref, f"{bits}-bit sparse n={n}")
        gh.compare_lse(lse[0], l_ref, f"{bits}-bit sparse n={n}")


@pytest.mark.parametrize("bits", WIDTHS)
def test_formats_ragged_steps(bits):
    """8 fused steps of the ragged paged batch (64 seeded lengths, permuted physical blocks); steps 0 and 7
    check every sequence's cache bytes and output, the others 4 watched sequences."""
    w = _w("ragged", bits)
    lens = [int(x) for x in wl.lengths(w)]
    steps = 8
    cap = max(lens) + steps + 64
    mb = -(-(cap - w.hot_tokens) // w.block_size)
    perm = wl.block_permutation(w, w.batch * mb).reshape(w.batch, mb)
    cache = gh.make_cache(w, cap, phys_ids=perm)
    gh.fill(cache, w, lens)
    watch = [0, 1, int(np.argmax(lens)), int(np.argmin(lens))]
    for step in range(steps):
        cur = [n + step for n in lens]
        q = wl.queries(w, step=step)
        out, lse = _fused(cache, w, cur, q)
        full = step in (0, steps - 1)
        seqs = list(range(w.batch)) if full else watch
        st = _states(w, [cur[b] + 1 for b in seqs], seqs)
        gh.check_state(cache, st, seqs)
        _compare(out, lse, q, st, f"{bits}-bit ragged step {step}", seqs)


def test_int4_long_config():
    """The 131072-token workload with 4-bit cold blocks: plain decode at 131071 tokens and the fused step
    to 131072 (the benchmarked plan), all 4 sequences' outputs and cache bytes against the oracle."""
    w = _w("long", 4)
    B = w.batch
    n0 = w.context - 1
    cache = gh.make_cache(w, w.context)
    q0, q1 = wl.queries(w), wl.queries(w, step=1)
    with oj.pool(B) as ex:
        futs = [ex.submit(oj.decode_job, "long", b, [n0, n0 + 1], [q0[b], q1[b]], n0 + 1, {"quant_bits": 4})
                for b in range(B)]
        gh.fill(cache, w, [n0] * B, chunk=8192)
        out0, lse0 = _decode(cache, q0)
        out1, lse1 = _fused(cache, w, [n0] * B, q1)
        codes, scales = cache.cold_codes(), cache.scale_array()
        for b, f in enumerate(futs):
            (r0, r1), st = f.result()
            gh.compare_out(out0[b], r0[0], f"int4 long seq {b} n={n0}")
            gh.compare_lse(lse0[b], r0[1], f"int4 long seq {b} n={n0}")
            gh.compare_out(out1[b], r1[0], f"int4 long seq {b} fused step")
            gh.compare_lse(lse1[b], r1[1], f"int4 long seq {b} fused step")
            gh.check_state(cache, [st], seqs=[b], codes=codes, scales=scales)
