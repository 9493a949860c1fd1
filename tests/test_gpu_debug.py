"""GPU parity of the debug statistics against the fp64 oracle, through the C ABI.

Hybrid KV Cache page 6.3 (kv_cache_debug: quantisation-error statistics) and KV Cache reuse page 6
(attention entropy).  quant_err[phys][h][K|V] = the largest |x - code * scale| of each coded tile:
the GPU takes each element's exact difference rounded once to fp32 (fma), so its maximum is the
fp32 rounding of the oracle's exact fp64 maximum, compared bit for bit.  entropy[b][hq] = -sum p ln p
of each query head's attention, from the kernel's fp32 online softmax: within 1e-3 of the oracle
(the same bound as lse, of which it is a difference).
"""
import dataclasses

import numpy as np
import pytest

import oracle.hkv_oracle as orc
import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu

ENT_MAX_ABS = 1e-3


def _w(name, bits, **kw):
    return dataclasses.replace(wl.WORKLOADS[name], name=f"{name}_dbg{bits}", quant_bits=bits, **kw)


def _check_qerr(cache, w, lens, qerr, what, seqs=None):
    seqs = list(range(len(lens))) if seqs is None else seqs
    got_all = qerr.cpu().numpy().reshape(cache.num_phys, cache.H, 2)
    hdr = cache.header_array()
    for b, n in zip(seqs, lens):
        k, v = gh.history(w, b, n)
        want = orc.quant_errors(k, v, w.hot_tokens, w.block_size, w.quant_bits).astype(np.float32)
        for j in range(want.shape[0]):
            got = got_all[int(hdr[b, j, 0])]
            assert np.array_equal(got.view(np.uint32), want[j].view(np.uint32)), (what, b, j, got, want[j])


def _check_entropy(ent, q, states, what, sels=None):
    got = ent.cpu().numpy()
    worst = 0.0
    for b, st in enumerate(states):
        want = orc.attention_entropy(q[b], st, None if sels is None else sels[b])
        d = float(np.max(np.abs(got[b] - want)))
        worst = max(worst, d)
        assert d <= ENT_MAX_ABS, f"{what} b={b}: entropy max abs {d}"
    gh.log(f"  {what}: entropy max|d|={worst:.2e}")


@pytest.mark.parametrize("bits", [8, 4, 0])
def test_debug_statistics(bits):
    """Bulk append (multi-block coder), one-token appends (single-pass coder, maximum kept or raised) and
    fused steps: every coded tile's error bit-exact; entropy of dense, sparse and fused decodes."""
    torch = gh.torch_mod()
    w = _w("llama8b", bits, batch=4)
    lens = [32 + 64 * 9 + 17, 32 + 64 * 3, 40, 32 + 64 * 20 + 63]
    cache = gh.make_cache(w, max(lens) + 80)
    qerr, ent = cache.enable_debug(w.n_q_heads)
    gh.fill(cache, w, lens)
    _check_qerr(cache, w, lens, qerr, f"{bits}-bit bulk")
    # one-token appends: the single-pass coder (in place when the maximum is kept)
    cur = list(lens)
    for step in range(5):
        gh.fill(cache, w, [n + 1 for n in cur], start=cur)
        cur = [n + 1 for n in cur]
    _check_qerr(cache, w, cur, qerr, f"{bits}-bit single-token appends")
    q = wl.queries(w, step=2)
    states = [orc.build_state(*gh.history(w, b, n), 32, 64, bits) for b, n in enumerate(cur)]
    qd = gh.upload(q)
    out = torch.empty_like(qd)
    cache.decode(qd, out=out)
    torch.cuda.synchronize()
    _check_entropy(ent, q, states, f"{bits}-bit dense")
    # sparse
    rng = np.random.default_rng(bits)
    sels = [rng.integers(0, max(1, s.n_cold), size=(w.n_kv_heads, 40)).astype(np.int32) for s in states]
    for s, sel in zip(states, sels):
        if s.n_cold == 0:
            sel[:] = -1
    ent.fill_(float("nan"))
    cache.decode(qd, out=out, sel_idx=gh.upload(np.stack(sels)), k_sel=40)
    torch.cuda.synchronize()
    _check_entropy(ent, q, states, f"{bits}-bit sparse", sels)
    # fused steps
    for step in range(3):
        kb = np.stack([wl.tokens(w, b, cur[b], 1, "k")[0] for b in range(w.batch)])
        vb = np.stack([wl.tokens(w, b, cur[b], 1, "v")[0] for b in range(w.batch)])
        ent.fill_(float("nan"))
        cache.append_decode(gh.upload(kb), gh.upload(vb), qd, out=out)
        torch.cuda.synchronize()
        cur = [n + 1 for n in cur]
        states = [orc.build_state(*gh.history(w, b, n), 32, 64, bits) for b, n in enumerate(cur)]
        _check_entropy(ent, q, states, f"{bits}-bit fused step {step}")
    _check_qerr(cache, w, cur, qerr, f"{bits}-bit fused steps")
    cache.close()


@pytest.mark.parametrize("d,g", [(64, 1), (64, 8), (128, 2), (128, 8)])
def test_debug_entropy_instances(d, g):
    """Entropy through the other (head_dim, group) instances, and with the statistics switched off the
    buffers are left untouched."""
    torch = gh.torch_mod()
    w = _w("tiny", 8, batch=2, n_q_heads=2 * g, head_dim=d)
    lens = [32 + 64 * 3 + 17, 32 + 64 * 6 + 40]
    cache = gh.make_cache(w, max(lens) + 64)
    qerr, ent = cache.enable_debug(w.n_q_heads)
    gh.fill(cache, w, lens)
    q = wl.queries(w, step=7)
    states = [orc.build_state(*gh.history(w, b, n), 32, 64) for b, n in enumerate(lens)]
    cache.decode(gh.upload(q))
    torch.cuda.synchronize()
    _check_entropy(ent, q, states, f"d={d} g={g}")
    _check_qerr(cache, w, lens, qerr, f"d={d} g={g}")
    cache.disable_debug()
    ent.fill_(-5.0)
    qerr.fill_(-5.0)
    cache.decode(gh.upload(q))
    gh.fill(cache, w, [n + 1 for n in lens], start=lens)
    torch.cuda.synchronize()
    assert bool((ent == -5.0).all()) and bool((qerr == -5.0).all())


def test_debug_entropy_claim_plan():
    """Entropy through a plan whose splits claim blocks (4 sequences of ~700 cold blocks) and through the
    no-allocation entry point."""
    import int8_kv_cache_hkv_amd as hkv
    torch = gh.torch_mod()
    w = _w("llama8b", 8, batch=4)
    lens = [32 + 64 * 700 + 9, 32 + 64 * 650, 32 + 64 * 699 + 63, 32 + 64 * 300 + 1]
    cache = gh.make_cache(w, max(lens) + 8)
    _, ent = cache.enable_debug(w.n_q_heads)
    gh.fill(cache, w, lens, chunk=8192)
    q = wl.queries(w, step=4)
    qd = gh.upload(q)
    cache.decode(qd)
    torch.cuda.synchronize()
    states = [orc.build_state(*gh.history(w, b, n), 32, 64) for b, n in enumerate(lens)]
    _check_entropy(ent, q, states, "claim plan")
    ent.fill_(float("nan"))
    out = torch.empty_like(qd)
    hkv.hkv_decode_attn_noalloc(cache.handle, cache.desc, qd, out)
    torch.cuda.synchronize()
    _check_entropy(ent, q, states, "claim plan, no-allocation entry point")
    cache.close()


def test_phase_stamps_are_ordered_and_change_nothing():
    """hkv_phase_stamps: every workgroup's start <= work done <= arrival, each (sequence, kv-head)
    merged once after its last arrival, the fused step's append phases in order; the outputs with
    and without timestamps are equal bit for bit (static plans)."""
    import int8_kv_cache_hkv_amd as hkv
    torch = gh.torch_mod()
    w = wl.WORKLOADS["llama8b"]
    n = 32 + 64 * 9 + 5
    B = 4
    caches = [gh.make_cache(w, n + 8, batch=B) for _ in range(2)]
    for c in caches:
        gh.fill(c, w, [n] * B)
    q = gh.upload(wl.queries(w)[:B])
    kb = gh.upload(np.stack([wl.tokens(w, b, n, 1, "k")[0] for b in range(B)]))
    vb = gh.upload(np.stack([wl.tokens(w, b, n, 1, "v")[0] for b in range(B)]))
    outs = []
    for use in (False, True):
        c = caches[int(use)]
        buf = torch.zeros(B * w.n_kv_heads * 140 * 8, dtype=torch.int64, device=q.device)
        if use:
            hkv.hkv_phase_stamps(c.handle, buf)
        o1 = torch.empty_like(q)
        c.decode(q, out=o1)
        torch.cuda.synchronize()
        st_plain = buf.cpu().numpy().copy()
        buf.zero_()
        o2 = torch.empty_like(q)
        c.append_decode(kb, vb, q, out=o2)
        torch.cuda.synchronize()
        st_fused = buf.cpu().numpy().copy()
        hkv.hkv_phase_stamps(c.handle, None)
        outs.append((o1.cpu().numpy(), o2.cpu().numpy()))
        if not use:
            assert not st_plain.any() and not st_fused.any()
            continue
        for st, fused in ((st_plain, False), (st_fused, True)):
            rows = st.reshape(-1, 8)
            npart = int((rows[:, 0] != 0).sum()) // (B * w.n_kv_heads)
            a = rows[:B * w.n_kv_heads * npart].reshape(B * w.n_kv_heads, npart, 8)
            assert (a[:, :, 0] > 0).all()
            assert (a[:, :, 0] <= a[:, :, 1]).all() and (a[:, :, 1] <= a[:, :, 2]).all()
            merges = (a[:, :, 3] != 0).sum(axis=1)
            assert (merges == 1).all(), "each (sequence, kv-head) merges once"
            assert (a[:, :, 3].max(axis=1) >= a[:, :, 1].max(axis=1)).all()
            if fused:
                app = a[:, npart - 1]
                assert (app[:, 0] <= app[:, 4]).all() and (app[:, 4] <= app[:, 6]).all()
                assert (app[:, 6] <= app[:, 7]).all() and (app[:, 7] <= app[:, 1]).all()
                coded = app[:, 5] != 0
                assert ((app[coded, 4] <= app[coded, 5]) & (app[coded, 5] <= app[coded, 6])).all()
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    for c in caches:
        c.close()
