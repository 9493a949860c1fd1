"""GPU parity of the HIP path against the fp64 oracle, through the C-ABI.

Bit-exact: INT8 codes, fp32 scales, block headers, hot ring and tail contents.
Within tolerance (max |d| <= 4e-3, mean |d| <= 5e-4 against fp64): the fp16
attention output.  Top-K: index sets equal outside near-ties of the K-th
window probability (|p - tau| <= 1e-5).
"""
import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh
from tests import oracle_jobs as oj

pytestmark = pytest.mark.gpu


def _decode(cache, q_np, lse=True, sel=None, k_sel=0):
    torch = gh.torch_mod()
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device) if lse else None
    cache.decode(q, out=out, lse=lse_t, sel_idx=sel, k_sel=k_sel)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse_t.cpu().numpy() if lse else None)


def _oracle_states(w, lens, seqs=None):
    seqs = list(range(len(lens))) if seqs is None else seqs
    out = []
    for b, n in zip(seqs, lens):
        k, v = gh.history(w, b, n)
        out.append(orc.build_state(k, v, w.hot_tokens, w.block_size, w.quant_bits))
    return out


# ------------------------------------------------------------------ tiny: every output, every byte
def test_tiny_config_parity():
    w = wl.WORKLOADS["tiny"]
    gh.log(f"tiny: B={w.batch} H={w.n_kv_heads} Hq={w.n_q_heads} d={w.head_dim} n={w.context}")
    cache = gh.make_cache(w, w.context)
    gh.fill(cache, w, [w.context])
    states = _oracle_states(w, [w.context])
    gh.check_state(cache, states)
    q = wl.queries(w)
    out, lse = _decode(cache, q)
    o_ref, l_ref = orc.decode(q[0], states[0])
    gh.compare_out(out[0], o_ref, "tiny out")
    gh.compare_lse(lse[0], l_ref, "tiny")


@pytest.mark.parametrize("n", [1, 5, 31, 32, 33, 95, 96, 97, 160, 161, 300])
def test_small_lengths_ragged_tail(n):
    """Empty/partial cold zones, exact block boundaries and ragged partial blocks."""
    w = wl.WORKLOADS["tiny"]
    cache = gh.make_cache(w, 400)
    gh.fill(cache, w, [n])
    states = _oracle_states(w, [n])
    gh.check_state(cache, states)
    q = wl.queries(w, step=n)
    out, lse = _decode(cache, q)
    o_ref, l_ref = orc.decode(q[0], states[0])
    gh.compare_out(out[0], o_ref, f"n={n}")
    gh.compare_lse(lse[0], l_ref, f"n={n}")


def test_append_chunking_invariance():
    """One bulk append, single-token appends and random chunks give identical bytes and outputs."""
    torch = gh.torch_mod()
    w = wl.WORKLOADS["tiny"]
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
        assert torch.equal(ref.cold, c.cold)
        assert torch.equal(ref.scales, c.scales)
        assert torch.equal(ref.headers, c.headers)
        assert torch.equal(ref.hot, c.hot)
    q = wl.queries(w, step=7)
    outs = [_decode(c, q)[0] for c in caches]
    assert all(np.array_equal(outs[0].view(np.uint16), o.view(np.uint16)) for o in outs[1:])
    gh.check_state(ref, _oracle_states(w, [n]))


# ------------------------------------------------------------------ Llama-3-8B-shaped layer, full size
def test_llama8b_config_parity():
    w = wl.WORKLOADS["llama8b"]
    gh.log(f"llama8b: B={w.batch} n={w.context} (K outliers x{w.outlier_scale})")
    cache = gh.make_cache(w, w.context + 64)
    gh.fill(cache, w, [w.context] * w.batch)
    states = _oracle_states(w, [w.context] * w.batch)
    gh.check_state(cache, states)
    q = wl.queries(w)
    out, lse = _decode(cache, q)
    o_ref = np.stack([orc.decode(q[b], states[b])[0] for b in range(w.batch)])
    l_ref = np.stack([orc.decode(q[b], states[b])[1] for b in range(w.batch)])
    gh.compare_out(out, o_ref, "llama8b out")
    gh.compare_lse(lse, l_ref, "llama8b")
    # one more decode step: append one token to every sequence (spill into the half block), decode again
    gh.fill(cache, w, [w.context + 1] * w.batch, start=[w.context] * w.batch)
    states = _oracle_states(w, [w.context + 1] * w.batch)
    gh.check_state(cache, states)
    q = wl.queries(w, step=1)
    out, _ = _decode(cache, q)
    o_ref = np.stack([orc.decode(q[b], states[b])[0] for b in range(w.batch)])
    gh.compare_out(out, o_ref, "llama8b step 1")


def test_decode_deterministic_and_permutation_invariant():
    """Two runs are bitwise equal; a different physical placement changes no output bit."""
    w = wl.WORKLOADS["llama8b"]
    n = 1000
    lens = [n] * 4
    mb = -(-(n + 10 - 32) // 64)
    a = gh.make_cache(w, n + 10, batch=4)
    perm = np.random.default_rng(3).permutation(4 * mb).reshape(4, mb)
    b = gh.make_cache(w, n + 10, batch=4, phys_ids=perm)
    gh.fill(a, w, lens)
    gh.fill(b, w, lens)
    q = wl.queries(w)[:4]
    o1, l1 = _decode(a, q)
    o2, l2 = _decode(a, q)
    o3, l3 = _decode(b, q)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16)) and np.array_equal(l1, l2)
    assert np.array_equal(o1.view(np.uint16), o3.view(np.uint16)) and np.array_equal(l1, l3)


# ------------------------------------------------------------------ ragged paged batch
def test_ragged_config_parity():
    w = wl.WORKLOADS["ragged"]
    lens = [int(x) for x in wl.lengths(w)]
    cap = max(lens) + w.steps + 64
    mb = -(-(cap - w.hot_tokens) // w.block_size)
    n_phys = w.batch * mb
    perm = wl.block_permutation(w, n_phys).reshape(w.batch, mb)
    gh.log(f"ragged: B={w.batch} lens {min(lens)}..{max(lens)} phys={n_phys} steps={w.steps}")
    cache = gh.make_cache(w, cap, phys_ids=perm)
    gh.fill(cache, w, lens)
    states = _oracle_states(w, lens)
    gh.check_state(cache, states)
    watch = [0, 1, int(np.argmax(lens)), int(np.argmin(lens))]
    for step in range(w.steps):
        cur = [n + step for n in lens]
        gh.fill(cache, w, [n + 1 for n in cur], start=cur)
        q = wl.queries(w, step=step)
        out, lse = _decode(cache, q)
        full = step in (0, w.steps - 1)
        seqs = list(range(w.batch)) if full else watch
        st = _oracle_states(w, [cur[b] + 1 for b in seqs], seqs)
        if full:
            gh.check_state(cache, st, seqs)
        o_ref = np.stack([orc.decode(q[b], s)[0] for b, s in zip(seqs, st)])
        gh.compare_out(out[seqs], o_ref, f"ragged step {step}")


# ------------------------------------------------------------------ fused one-token append + decode
def _step_tokens(w, cur):
    """The token at position cur[b] of every sequence b: K and V fp16 [B, H, D]."""
    kb = np.stack([wl.tokens(w, b, cur[b], 1, "k")[0] for b in range(len(cur))])
    vb = np.stack([wl.tokens(w, b, cur[b], 1, "v")[0] for b in range(len(cur))])
    return kb, vb


def _append_decode(cache, w, cur, q_np):
    torch = gh.torch_mod()
    kb, vb = _step_tokens(w, cur)
    q = gh.upload(q_np)
    out = torch.empty_like(q)
    lse_t = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    cache.append_decode(gh.upload(kb), gh.upload(vb), q, out=out, lse=lse_t)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse_t.cpu().numpy()


@pytest.mark.parametrize("n0", [0, 5, 31, 32, 33, 40, 95, 96, 97, 159, 160, 161, 287, 300])
def test_append_decode_small(n0):
    """One fused step from lengths where the hot zone is not full, where the spilled token opens a
    block, lands inside one (maximum kept or raised) or completes one."""
    w = wl.WORKLOADS["tiny"]
    cache = gh.make_cache(w, 400)
    gh.fill(cache, w, [n0])
    q = wl.queries(w, step=n0)
    out, lse = _append_decode(cache, w, [n0], q)
    st = _oracle_states(w, [n0 + 1])
    gh.check_state(cache, st)
    o_ref, l_ref = orc.decode(q[0], st[0])
    gh.compare_out(out[0], o_ref, f"fused n0={n0} out")
    gh.compare_lse(lse[0], l_ref, f"fused n0={n0}")


def test_append_decode_ragged_steps():
    """16 fused steps over the ragged paged batch (permuted physical blocks): cache state and output
    against the oracle after every step."""
    w = wl.WORKLOADS["ragged"]
    lens = [int(x) for x in wl.lengths(w)]
    steps = 16
    cap = max(lens) + steps + 64
    mb = -(-(cap - w.hot_tokens) // w.block_size)
    n_phys = w.batch * mb
    perm = wl.block_permutation(w, n_phys).reshape(w.batch, mb)
    cache = gh.make_cache(w, cap, phys_ids=perm)
    gh.fill(cache, w, lens)
    watch = [0, 1, int(np.argmax(lens)), int(np.argmin(lens))]
    for step in range(steps):
        cur = [n + step for n in lens]
        q = wl.queries(w, step=step)
        out, _ = _append_decode(cache, w, cur, q)
        full = step in (0, steps - 1)
        seqs = list(range(w.batch)) if full else watch
        st = _oracle_states(w, [cur[b] + 1 for b in seqs], seqs)
        gh.check_state(cache, st, seqs)
        o_ref = np.stack([orc.decode(q[b], s)[0] for b, s in zip(seqs, st)])
        gh.compare_out(out[seqs], o_ref, f"fused ragged step {step}")


@pytest.mark.parametrize("batch", [256, 260])
def test_append_decode_length_protocols(batch):
    """Fused steps over 256 sequences (lengths from the launch arguments, one store per sequence
    publishes the new length) and over 260 (more than the launch arguments hold: seq_len read on the
    device, the last of the H merges of a sequence publishes it).  Three steps; after each, every
    device length is the host mirror's, and sampled sequences' outputs and cache state equal the
    oracle's."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["tiny"], batch=batch)
    lens = [20 + (37 * b) % 380 for b in range(batch)]
    cache = gh.make_cache(w, 460, batch=batch)
    gh.fill(cache, w, lens)
    watch = [0, 1, batch // 2, batch - 1]
    for step in range(3):
        cur = [n + step for n in lens]
        q = wl.queries(w, step=step)
        out, lse = _append_decode(cache, w, cur, q)
        assert cache.seq_len.cpu().numpy().tolist() == [n + 1 for n in cur]
        assert cache.seq_len_host.tolist() == [n + 1 for n in cur]
        st = _oracle_states(w, [cur[b] + 1 for b in watch], watch)
        gh.check_state(cache, st, watch)
        for b, s in zip(watch, st):
            o_ref, l_ref = orc.decode(q[b], s)
            gh.compare_out(out[b], o_ref, f"fused batch {batch} step {step} seq {b}")
            gh.compare_lse(lse[b], l_ref, f"fused batch {batch} step {step} seq {b}")


def test_append_decode_equals_separate_calls():
    """The fused step leaves the same cache bytes as hkv_append + hkv_decode_attn, and the outputs
    agree (different split plans: equal to the tolerance, not bitwise)."""
    w = wl.WORKLOADS["llama8b"]
    n0 = w.context - 1
    a = gh.make_cache(w, n0 + 8)
    b = gh.make_cache(w, n0 + 8)
    gh.fill(a, w, [n0] * w.batch)
    gh.fill(b, w, [n0] * w.batch)
    q = wl.queries(w, step=3)
    out_f, lse_f = _append_decode(a, w, [n0] * w.batch, q)
    gh.fill(b, w, [n0 + 1] * w.batch, start=[n0] * w.batch)
    out_s, lse_s = _decode(b, q)
    assert np.array_equal(a.cold_codes(), b.cold_codes())
    assert np.array_equal(a.scale_array(), b.scale_array())
    assert np.array_equal(a.header_array(), b.header_array())
    assert np.array_equal(a.hot_array(), b.hot_array())
    assert np.array_equal(a.tail.cpu().numpy(), b.tail.cpu().numpy())
    assert np.array_equal(a.seq_len.cpu().numpy(), b.seq_len.cpu().numpy())
    gh.compare_out(out_f.astype(np.float64), out_s.astype(np.float64), "fused vs separate")
    assert np.max(np.abs(lse_f - lse_s)) <= gh.LSE_MAX_ABS


# ------------------------------------------------------------------ quantiser edge values
def _edge_history(H=2, d=64, seed=5):
    """Four cold blocks (all zero; exact half-integer ratios x/s with s = 1; fp16 extremes and
    subnormals; random) followed by random hot tokens, as one sequence history [n, H, d]."""
    rng = np.random.default_rng(seed)
    S, T = 64, 32
    blocks = []
    blocks.append(np.zeros((S, H, d), dtype=np.float16))
    half = (rng.integers(-127, 127, size=(S, H, d)) + 0.5).astype(np.float16)  # x / 1.0 = k + 0.5: a tie
    half[0, :, 0] = 127.0                                                   # the maximum: s = fl32(127/127) = 1
    blocks.append(half)
    ext = rng.standard_normal((S, H, d)).astype(np.float16)
    ext[:, :, ::3] = np.float16(6e-8)       # fp16 subnormals
    ext[:, :, 1::7] = np.float16(-65504.0)  # fp16 extremes
    ext[5, :, 2] = np.float16(65504.0)
    blocks.append(ext)
    blocks.append(rng.standard_normal((S, H, d)).astype(np.float16))
    cold = np.concatenate(blocks)
    hot = rng.standard_normal((T, H, d)).astype(np.float16)
    return np.concatenate([cold, hot])


def test_quantiser_edge_values():
    """Zero blocks (scale 0), exact ties of x / s (round half to even), fp16 extremes and subnormals:
    codes and scales bit-exact, decode within tolerance; then one fused step spilling an extreme token."""
    torch = gh.torch_mod()
    import int8_kv_cache_hkv_amd as hkv
    H, d = 2, 64
    hist = _edge_history(H, d)
    vals = _edge_history(H, d, seed=6)
    n = hist.shape[0]
    cache = hkv.HybridKVCache(H, d, 1, n + 64)
    cache.append(gh.upload(hist[None]), gh.upload(vals[None]))
    torch.cuda.synchronize()
    st = orc.build_state(hist, vals, 32, 64)
    gh.check_state(cache, [st])
    q = np.random.default_rng(7).standard_normal((1, 2 * H, d)).astype(np.float16) * np.float16(0.01)
    out, lse = _decode(cache, q)
    o_ref, l_ref = orc.decode(q[0], st)
    gh.compare_out(out[0], o_ref, "edge values")
    gh.compare_lse(lse[0], l_ref, "edge values")
    # one fused step: the spilled token opens a fifth block; the new token holds an fp16 extreme
    kn = np.random.default_rng(8).standard_normal((1, H, d)).astype(np.float16)
    kn[0, 0, 3] = np.float16(65504.0)
    out_f = torch.empty((1, 2 * H, d), dtype=torch.float16, device="cuda")
    cache.append_decode(gh.upload(kn), gh.upload(kn), gh.upload(q), out=out_f)
    torch.cuda.synchronize()
    st1 = orc.build_state(np.concatenate([hist, kn]), np.concatenate([vals, kn]), 32, 64)
    gh.check_state(cache, [st1])
    o_ref1, _ = orc.decode(q[0], st1)
    gh.compare_out(out_f.cpu().numpy()[0], o_ref1, "edge values, fused step")


# ------------------------------------------------------------------ every (head_dim, group) instance
@pytest.mark.parametrize("d,g", [(64, 1), (64, 8), (128, 1), (128, 2), (128, 4), (128, 8)])
def test_group_sizes_dense_sparse_fused(d, g):
    """Every built (head_dim, GQA group) instance of the decode kernel, plain, sparse and fused, on two
    sequences of different lengths (each with a ragged tail block) against the oracle."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["tiny"], name=f"gqa_d{d}_g{g}", batch=2, n_q_heads=2 * g, head_dim=d)
    lens = [32 + 64 * 3 + 17, 32 + 64 * 6 + 40]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=7)
    st = _oracle_states(w, lens)
    out, lse = _decode(cache, q)
    for b in range(2):
        o_ref, l_ref = orc.decode(q[b], st[b])
        gh.compare_out(out[b], o_ref, f"d={d} g={g} dense b={b}")
        gh.compare_lse(lse[b], l_ref, f"d={d} g={g} dense b={b}")
    k_sel = 50
    rng = np.random.default_rng(10 * d + g)
    sel = np.stack([rng.integers(0, s.n_cold, size=(w.n_kv_heads, k_sel)) for s in st]).astype(np.int32)
    out_s, lse_s = _decode(cache, q, sel=gh.upload(sel), k_sel=k_sel)
    for b in range(2):
        o_ref, l_ref = orc.sparse_decode(q[b], st[b], sel[b])
        gh.compare_out(out_s[b], o_ref, f"d={d} g={g} sparse b={b}")
        gh.compare_lse(lse_s[b], l_ref, f"d={d} g={g} sparse b={b}")
    out_f, lse_f = _append_decode(cache, w, lens, q)
    st1 = _oracle_states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    for b in range(2):
        o_ref, l_ref = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"d={d} g={g} fused b={b}")
        gh.compare_lse(lse_f[b], l_ref, f"d={d} g={g} fused b={b}")


# ------------------------------------------------------------------ other hot-zone sizes
@pytest.mark.parametrize("T", [16, 64, 128])
def test_hot_tokens_variants(T):
    """hot_tokens 16, 64 and 128 (the other protocol values): bulk append, dense decode, a fused step,
    top-K and sparse decode against the oracle; one sequence with a cold zone, one still all-hot."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["tiny"], name=f"hot{T}", batch=2, hot_tokens=T)
    lens = [T + 64 * 3 + 17, T - 5]
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens)
    st = _oracle_states(w, lens)
    gh.check_state(cache, st)
    q = wl.queries(w, step=1)
    out, lse = _decode(cache, q)
    for b in range(2):
        o_ref, l_ref = orc.decode(q[b], st[b])
        gh.compare_out(out[b], o_ref, f"T={T} dense b={b}")
        gh.compare_lse(lse[b], l_ref, f"T={T} dense b={b}")
    k = 50
    idx = cache.topk(gh.upload(q), k)
    gh.torch_mod().cuda.synchronize()
    got = idx.cpu().numpy()
    want, pr, tau = orc.topk_select(q[0], st[0], k)
    for h in range(w.n_kv_heads):
        gh.compare_topk(got[0, h], want[h], pr[h], tau[h], st[0].n_cold, k, f"T={T} topk h={h}")
    out_s, lse_s = _decode(cache, q, sel=idx, k_sel=k)
    for b in range(2):
        o_ref, l_ref = orc.sparse_decode(q[b], st[b], got[b])
        gh.compare_out(out_s[b], o_ref, f"T={T} sparse b={b}")
    out_f, _ = _append_decode(cache, w, lens, q)
    st1 = _oracle_states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    for b in range(2):
        o_ref, _ = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"T={T} fused b={b}")


# ------------------------------------------------------------------ XCD-major order on a grid not a multiple of 8
def test_claim_walk_odd_grid():
    """3 sequences x 3 kv-heads with ~86k tokens: a resident plan with long splits, so the waves claim
    their blocks dynamically and the grid is read in the rotated split-major order over 9 (sequence,
    kv-head) pairs, with a workgroup count that is not a multiple of the 8 dies.  Every output
    against the oracle, plain decode and a fused step."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["long"], name="claim_odd", batch=3, n_kv_heads=3, n_q_heads=6)
    n = 32 + 1345 * 64 + 17
    cache = gh.make_cache(w, n + 8)
    gh.fill(cache, w, [n] * w.batch, chunk=8192)
    q = wl.queries(w, step=2)
    out, lse = _decode(cache, q)
    st = _oracle_states(w, [n] * w.batch)
    for b in range(w.batch):
        o_ref, l_ref = orc.decode(q[b], st[b])
        gh.compare_out(out[b], o_ref, f"claim odd grid b={b}")
        gh.compare_lse(lse[b], l_ref, f"claim odd grid b={b}")
    out_f, _ = _append_decode(cache, w, [n] * w.batch, q)
    st1 = _oracle_states(w, [n + 1] * w.batch)
    for b in range(w.batch):
        o_ref, _ = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"claim odd grid fused b={b}")


def test_claim_walk_ragged_batch():
    """32 sequences x 8 kv-heads, lengths from 40 tokens to 100 cold blocks, blocks at a permuted
    physical placement: the resident plan has splits of at least 16 blocks, so after their first
    block the waves claim blocks from the per-(sequence, kv-head) counters.  Sequences with fewer
    blocks than the static first round (every claim lands past the end), with exactly one claimable
    block, and with many.  Plain decode twice (the second call finds the counters back at zero),
    then a fused step; every output against the oracle."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["llama8b"], name="claim", batch=32)
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
    st = _oracle_states(w, lens)
    for b in range(w.batch):
        o_ref, l_ref = orc.decode(q[b], st[b])
        for o, l, tag in ((o1, l1, "first"), (o2, l2, "second")):
            gh.compare_out(o[b], o_ref, f"claim {tag} b={b} n={lens[b]}")
            gh.compare_lse(l[b], l_ref, f"claim {tag} b={b}")
    out_f, lse_f = _append_decode(cache, w, lens, q)
    st1 = _oracle_states(w, [n + 1 for n in lens])
    for b in range(w.batch):
        o_ref, l_ref = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"claim fused b={b} n={lens[b]}")
        gh.compare_lse(lse_f[b], l_ref, f"claim fused b={b}")


@pytest.mark.parametrize("d,g", [(64, 1), (64, 8), (128, 1), (128, 2), (128, 8)])
def test_claim_walk_group_sizes(d, g):
    """The claim walk in every other built (head_dim, GQA group) instance (d = 128, G = 4 runs in the
    tests above): 16 sequences x 8 kv-heads of 70 to 95 cold blocks, so the plain and the fused plan
    both have splits of at least 16 blocks; plain decode and a fused step against the oracle."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["llama8b"], name=f"claim_d{d}_g{g}", batch=16, n_kv_heads=8,
                            n_q_heads=8 * g, head_dim=d)
    rng = np.random.default_rng(100 * d + g)
    lens = (32 + 64 * rng.integers(70, 96, w.batch) + rng.integers(0, 64, w.batch)).tolist()
    lens[0] = 32 + 64 * 95 + 5  # the longest sequence sets the plan: splits of 32 (plain) / 48 (fused) blocks
    cache = gh.make_cache(w, max(lens) + 8)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=3)
    out, lse = _decode(cache, q)
    st = _oracle_states(w, lens)
    for b in range(w.batch):
        o_ref, l_ref = orc.decode(q[b], st[b])
        gh.compare_out(out[b], o_ref, f"claim d={d} g={g} b={b}")
        gh.compare_lse(lse[b], l_ref, f"claim d={d} g={g} b={b}")
    out_f, lse_f = _append_decode(cache, w, lens, q)
    st1 = _oracle_states(w, [n + 1 for n in lens])
    for b in range(w.batch):
        o_ref, l_ref = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"claim fused d={d} g={g} b={b}")
        gh.compare_lse(lse_f[b], l_ref, f"claim fused d={d} g={g} b={b}")


@pytest.mark.parametrize("batch", [200, 300])
def test_batch_plan_orders(batch):
    """Batch plans (more (sequence, kv-head) pairs than resident slots): 200 sequences x 2 kv-heads fit
    the longest-first order table (400 groups), 300 do not (600 groups: sequence order).  Lengths
    40..420 tokens; plain decode and a fused step, every output against the oracle."""
    import dataclasses
    w = dataclasses.replace(wl.WORKLOADS["tiny"], name=f"batch{batch}", batch=batch)
    rng = np.random.default_rng(batch)
    lens = rng.integers(40, 421, batch).tolist()
    cache = gh.make_cache(w, max(lens) + 8)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=5)
    out, lse = _decode(cache, q)
    st = _oracle_states(w, lens)
    for b in range(batch):
        o_ref, l_ref = orc.decode(q[b], st[b])
        gh.compare_out(out[b], o_ref, f"batch {batch} b={b}")
        gh.compare_lse(lse[b], l_ref, f"batch {batch} b={b}")
    out_f, lse_f = _append_decode(cache, w, lens, q)
    st1 = _oracle_states(w, [n + 1 for n in lens])
    gh.check_state(cache, st1)
    for b in range(batch):
        o_ref, l_ref = orc.decode(q[b], st1[b])
        gh.compare_out(out_f[b], o_ref, f"batch {batch} fused b={b}")
        gh.compare_lse(lse_f[b], l_ref, f"batch {batch} fused b={b}")


# ------------------------------------------------------------------ long context, every sequence
def test_long_config_parity():
    """The 131072-token workload at full size: a plain decode at 131071 tokens, then the fused step
    (append one token + decode, the launch plan the benchmark times) to 131072 tokens, then a plain
    decode there; out and lse of all 4 sequences against the oracle after each, and every block's
    codes, scales, headers and the hot ring of all 4 sequences bit-exact after the fused step."""
    w = wl.WORKLOADS["long"]
    B = w.batch
    n0 = w.context - 1
    gh.log(f"long: B={B} n0={n0} -> {n0 + 1} (fused step)")
    cache = gh.make_cache(w, w.context)
    q0, q1 = wl.queries(w), wl.queries(w, step=1)
    with oj.pool(B) as ex:
        futs = [ex.submit(oj.decode_job, "long", b, [n0, n0 + 1], [q0[b], q1[b]], n0 + 1) for b in range(B)]
        gh.fill(cache, w, [n0] * B, chunk=8192)
        out0, lse0 = _decode(cache, q0)
        out1, lse1 = _append_decode(cache, w, [n0] * B, q1)
        out2, lse2 = _decode(cache, q1)
        codes, scales = cache.cold_codes(), cache.scale_array()
        for b, f in enumerate(futs):
            (r0, r1), st = f.result()
            gh.log(f"  long seq {b}: oracle done")
            gh.compare_out(out0[b], r0[0], f"long seq {b} n={n0}")
            gh.compare_lse(lse0[b], r0[1], f"long seq {b} n={n0}")
            gh.compare_out(out1[b], r1[0], f"long seq {b} fused step")
            gh.compare_lse(lse1[b], r1[1], f"long seq {b} fused step")
            gh.compare_out(out2[b], r1[0], f"long seq {b} n={n0 + 1}")
            gh.compare_lse(lse2[b], r1[1], f"long seq {b} n={n0 + 1}")
            gh.check_state(cache, [st], seqs=[b], codes=codes, scales=scales)


# ------------------------------------------------------------------ top-K and sparse decode
@pytest.mark.parametrize("n,k", [(32 + 100, 128), (32 + 300, 50), (32 + 64 * 9 + 17, 100), (20, 16),
                                 # rows at and just past the register-resident selection limit (32768 keys)
                                 (32 + 32768, 512), (32 + 32769, 512), (32 + 40007, 300)])
def test_topk_small(n, k):
    w = wl.WORKLOADS["tiny"]
    cache = gh.make_cache(w, n + 64)
    gh.fill(cache, w, [n])
    st = _oracle_states(w, [n])[0]
    q = wl.queries(w, step=3)
    idx = cache.topk(gh.upload(q), k)
    gh.torch_mod().cuda.synchronize()
    got = idx.cpu().numpy()
    want, p, tau = orc.topk_select(q[0], st, k)
    for h in range(w.n_kv_heads):
        gh.compare_topk(got[0, h], want[h], p[h], tau[h], st.n_cold, k, f"n={n} k={k} h={h}")
    if st.n_cold > 0:
        out, lse = _decode(cache, q, sel=idx, k_sel=k)
        o_ref, l_ref = orc.sparse_decode(q[0], st, got[0])
        gh.compare_out(out[0], o_ref, "sparse")
        gh.compare_lse(lse[0], l_ref, "sparse")


@pytest.mark.parametrize("k", [512, 100, 1])
def test_topk_ragged_rows(k):
    """One batch whose rows take every selection path: at most K keys (identity), rows of up to 8192
    keys (one workgroup, keys from the row), and longer rows split into 4096-key chunks that hand
    their candidates above a floor to the row's last workgroup (8193 keys: a 1-key last chunk;
    20000 and 40017 keys: several chunks).  Every row's index set against the oracle."""
    w = wl.WORKLOADS["tiny"]
    lens = [32 + 100, 32 + 600, 32 + 8192, 32 + 8193, 32 + 20000, 32 + 40017]
    import dataclasses
    w = dataclasses.replace(w, batch=len(lens))
    cache = gh.make_cache(w, max(lens) + 64)
    gh.fill(cache, w, lens, chunk=8192)
    states = _oracle_states(w, lens)
    q = wl.queries(w, step=4)
    idx = cache.topk(gh.upload(q), k)
    gh.torch_mod().cuda.synchronize()
    got = idx.cpu().numpy()
    for b, st in enumerate(states):
        want, p, tau = orc.topk_select(q[b], st, k)
        for h in range(w.n_kv_heads):
            gh.compare_topk(got[b, h], want[h], p[h], tau[h], st.n_cold, k, f"n={lens[b]} k={k} b={b} h={h}")
    # the same workspace again: the chunk arrival counters are back at zero
    idx2 = cache.topk(gh.upload(q), k).cpu().numpy()
    assert np.array_equal(idx2, got)


@pytest.mark.parametrize("k_sel", [1, 15, 16, 17, 37, 64, 100])
def test_sparse_decode_explicit_indices(k_sel):
    """Caller-built selections: ragged k_sel, -1 and out-of-range entries are ignored, duplicates count twice."""
    w = wl.WORKLOADS["tiny"]
    n = 32 + 64 * 5 + 9
    cache = gh.make_cache(w, n + 64)
    gh.fill(cache, w, [n])
    st = _oracle_states(w, [n])[0]
    q = wl.queries(w, step=5)
    rng = np.random.default_rng(1000 + k_sel)
    sel = rng.integers(0, st.n_cold, size=(1, w.n_kv_heads, k_sel)).astype(np.int32)
    m = rng.random(sel.shape)
    sel[m < 0.1] = -1
    sel[(m >= 0.1) & (m < 0.14)] = st.n_cold + 7
    sel[(m >= 0.14) & (m < 0.17)] = 2 ** 31 - 1
    out, lse = _decode(cache, q, sel=gh.upload(sel), k_sel=k_sel)
    ref_sel = np.where((sel[0] >= 0) & (sel[0] < st.n_cold), sel[0], -1)
    o_ref, l_ref = orc.sparse_decode(q[0], st, ref_sel)
    gh.compare_out(out[0], o_ref, f"sparse explicit k_sel={k_sel}")
    gh.compare_lse(lse[0], l_ref, f"sparse explicit k_sel={k_sel}")


@pytest.mark.parametrize("n,k", [(32 + 64 * 4, 10), (32 + 32768, 512), (32 + 32768 - 5, 300)])
def test_topk_ties_prefer_lower_index(n, k):
    """Identical keys tie exactly in fp32 too: the lowest token indices must be chosen (short rows,
    and full register-resident rows where the selection first narrows to keys above a floor)."""
    torch = gh.torch_mod()
    import int8_kv_cache_hkv_amd as hkv
    H, D = 2, 64
    cache = hkv.HybridKVCache(H, D, 1, n)
    kv = np.ones((1, n, H, D), dtype=np.float16)
    cache.append(gh.upload(kv), gh.upload(kv))
    q = np.ones((1, 2 * H, D), dtype=np.float16)
    idx = cache.topk(gh.upload(q), k)
    torch.cuda.synchronize()
    # every cosine is 1, so a token's window probability is 1 / (valid tokens of its window): a
    # short last window ranks first, then the lowest indices
    n_cold = n - 32
    p = np.array([1.0 / min(64, n_cold - (t // 64) * 64) for t in range(n_cold)])
    want = sorted(sorted(range(n_cold), key=lambda t: (-p[t], t))[:k])
    assert idx.cpu().numpy()[0].tolist() == [want] * H


@pytest.mark.parametrize("flat,k", [(tuple(range(12)), 180),
                                    (tuple(range(12)) + tuple(range(64, 70)), 200),
                                    ((3, 63, 64, 127, 159), 170)])
def test_topk_whole_windows(flat, k):
    """Windows whose every top clears the floor are read whole (by their wave, one key per lane):
    a row of 160 windows where the `flat` windows hold 64 equal keys (probability 1/64 each) and
    every other window one key aligned with the query and 63 opposed ones (1/(1 + 63/e^2) and
    that / e^2), with K between the aligned keys and the flat ones.  Covers more whole windows in
    one wave than it keeps in registers, whole windows in two waves, and the one-wave and workgroup
    selections of the candidates (916, 1294 and 475 of them).  Exact index set (equal keys tie exactly:
    the lowest indices), and the oracle's."""
    import int8_kv_cache_hkv_amd as hkv
    torch = gh.torch_mod()
    H, D, T, S, nw = 2, 64, 32, 64, 160
    n_cold = S * nw
    n = n_cold + T
    kv = -np.ones((1, n, H, D), dtype=np.float16)
    for wi in range(nw):
        if wi in flat:
            kv[0, S * wi:S * (wi + 1)] = 1
        else:
            kv[0, S * wi + 5] = 1
    kv[0, n_cold:] = 1
    cache = hkv.HybridKVCache(H, D, 1, n)
    cache.append(gh.upload(kv), gh.upload(kv))
    q = np.ones((1, 2 * H, D), dtype=np.float16)
    idx = cache.topk(gh.upload(q), k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()[0]
    aligned = [S * wi + 5 for wi in range(nw) if wi not in flat]
    flat_tokens = [t for wi in sorted(flat) for t in range(S * wi, S * (wi + 1))]
    want = sorted(aligned + flat_tokens[:k - len(aligned)])
    assert got.tolist() == [want] * H
    st = orc.build_state(kv[0], kv[0], T, S)
    w_or, p, tau = orc.topk_select(q[0], st, k)
    for h in range(H):
        assert w_or[h].tolist() == want
        gh.compare_topk(got[h], w_or[h], p[h], tau[h], st.n_cold, k, f"whole windows {flat} k={k} h={h}")


@pytest.mark.parametrize("n_uniform,k", [(3, 505), (4, 510)])
def test_topk_whole_windows_above_floor_bin(n_uniform, k):
    """The K-th largest key above the floor's bin: `n_uniform` windows of 64 equal keys (1/64 each,
    whole) among windows of 3 keys aligned with the query, 2 keys at cosine -0.9 and 59 opposed ones
    (0.0886, 0.0133, 0.0120).  The K-th largest window top is a 0.0133 key, so the floor sits there,
    but the uniform windows' keys put tau at 1/64, above its bin: the selection searches the whole
    candidate range (977 candidates: one wave; 1036: the workgroup).  Exact index set, and the
    oracle's."""
    import int8_kv_cache_hkv_amd as hkv
    torch = gh.torch_mod()
    H, D, T, S, nw = 2, 64, 32, 64, 160
    n_cold = S * nw
    n = n_cold + T
    alt = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)
    uniform = list(range(0, nw, nw // n_uniform))[:n_uniform]
    kv = -np.ones((1, n, H, D), dtype=np.float16)
    for wi in range(nw):
        base = S * wi
        if wi in uniform:
            kv[0, base:base + S] = 1
        else:
            kv[0, base:base + 3] = 1
            kv[0, base + 3:base + 5] = (-0.9 + 0.436 * alt).astype(np.float16)
    kv[0, n_cold:] = 1
    cache = hkv.HybridKVCache(H, D, 1, n)
    cache.append(gh.upload(kv), gh.upload(kv))
    q = np.ones((1, 2 * H, D), dtype=np.float16)
    idx = cache.topk(gh.upload(q), k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()[0]
    aligned = [S * wi + j for wi in range(nw) if wi not in uniform for j in range(3)]
    flat_tokens = [S * wi + j for wi in uniform for j in range(S)]
    want = sorted(aligned + flat_tokens[:k - len(aligned)])
    assert got.tolist() == [want] * H
    st = orc.build_state(kv[0], kv[0], T, S)
    w_or, p, tau = orc.topk_select(q[0], st, k)
    for h in range(H):
        assert w_or[h].tolist() == want
        gh.compare_topk(got[h], w_or[h], p[h], tau[h], st.n_cold, k, f"above the floor's bin k={k} h={h}")


def test_topk_config_parity():
    """The 32768-token top-K workload at full size: the index sets of all 16 sequences x 8 kv-heads
    and the sparse decode over each selection against the oracle; then a dense decode and a second
    selection on the same workspace (the claim counters must be back at zero)."""
    w = wl.WORKLOADS["topk"]
    n = w.context
    B = w.batch
    gh.log(f"topk: B={B} n={n} K={w.k_sel}")
    cache = gh.make_cache(w, n)
    gh.fill(cache, w, [n] * B, chunk=8192)
    q = wl.queries(w)
    qd = gh.upload(q)
    idx = cache.topk(qd, w.k_sel)
    out, lse = _decode(cache, q, sel=idx, k_sel=w.k_sel)
    got = idx.cpu().numpy()
    out_d, lse_d = _decode(cache, q)
    idx2 = cache.topk(qd, w.k_sel).cpu().numpy()
    assert np.array_equal(idx2, got), "top-K differs after a dense decode on the same workspace"
    with oj.pool(B) as ex:
        futs = [ex.submit(oj.topk_job, "topk", b, q[b], w.k_sel, got[b]) for b in range(B)]
        dense = [ex.submit(oj.decode_job, "topk", b, [n], [q[b]]) for b in (0, B - 1)]
        for b, f in enumerate(futs):
            want, p, tau, n_cold, o_ref, l_ref = f.result()
            for h in range(w.n_kv_heads):
                gh.compare_topk(got[b, h], want[h], p[h], tau[h], n_cold, w.k_sel, f"topk b={b} h={h}")
            gh.compare_out(out[b], o_ref, f"sparse b={b}")
            gh.compare_lse(lse[b], l_ref, f"sparse b={b}")
        for b, f in zip((0, B - 1), dense):
            ((o_ref, l_ref),), _ = f.result()
            gh.compare_out(out_d[b], o_ref, f"dense after top-K b={b}")
            gh.compare_lse(lse_d[b], l_ref, f"dense after top-K b={b}")
