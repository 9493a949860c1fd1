"""Independent checks that pin the fp64 oracle to the pages and to mathematics.

Nothing here re-types the oracle's formulas: scales and codes are checked
against exact rational arithmetic (``fractions.Fraction`` with integer
rounding written out below), attention against torch's
``scaled_dot_product_attention`` in float64 and against explicit Python
loops, top-K against a brute-force sort, and metadata sizing against the
worked example printed on the Hybrid KV Cache page (section 5.4).

Each ``pin_*`` function raises AssertionError on a mismatch; the test module
runs them on the real oracle and, with planted mistakes, shows that each
plausible slip in the oracle trips at least one pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction
from typing import List, Tuple

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- exact helpers
def fp32_nearest(fr: Fraction) -> float:
    """Round a rational to the nearest IEEE binary32 value, ties to even, using integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1.0 if fr < 0 else 1.0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # normalise so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, -149)                 # quantum: 24-bit significand, subnormals below 2^-126
    scaled = a / (Fraction(2) ** q)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(n) * 2.0 ** q


def round_half_even(x: float) -> int:
    n = math.floor(x)
    r = x - n
    if r > 0.5 or (r == 0.5 and n % 2 == 1):
        n += 1
    return int(n)


def exact_scale(tile: np.ndarray, lim: int = 127) -> float:
    m = max((abs(Fraction(float(v))) for v in np.asarray(tile, dtype=np.float16).ravel()), default=Fraction(0))
    return fp32_nearest(m / lim)


def exact_code(x: float, s: float, lim: int = 127) -> int:
    if s == 0.0:
        return 0
    quot = fp32_nearest(Fraction(float(x)) / Fraction(s))
    return max(-lim, min(lim, round_half_even(quot)))


# largest code magnitude per cold-zone width (written out, not taken from the oracle)
LIMIT = {8: 127, 4: 7}


def brute_history_kv(k_hist, v_hist, hot: int, block: int, h: int, bits: int = 8) -> Tuple[List, List]:
    """Key/value rows of kv-head h that decode attends to, built with exact arithmetic and loops
    (bits 0: the cold rows are the fp16 values themselves)."""
    n = len(k_hist)
    n_hot = min(n, hot)
    n_cold = n - n_hot
    keys, vals = [], []
    j = 0
    while j * block < n_cold:
        rows = range(j * block, min((j + 1) * block, n_cold))
        for src, dst in ((k_hist, keys), (v_hist, vals)):
            tile = np.array([[src[t][h][c] for c in range(src.shape[2])] for t in rows], dtype=np.float16)
            if bits == 0:
                for t in range(tile.shape[0]):
                    dst.append([float(x) for x in tile[t]])
                continue
            lim = LIMIT[bits]
            s = exact_scale(tile, lim)
            for t in range(tile.shape[0]):
                dst.append([float(exact_code(float(x), s, lim)) * s for x in tile[t]])
        j += 1
    for t in range(n_cold, n):
        keys.append([float(x) for x in k_hist[t][h]])
        vals.append([float(x) for x in v_hist[t][h]])
    return keys, vals


def brute_attend(q_row, keys, vals):
    d = len(q_row)
    z = [sum(q_row[c] * k[c] for c in range(d)) / math.sqrt(d) for k in keys]
    zm = max(z)
    e = [math.exp(v - zm) for v in z]
    den = sum(e)
    out = [sum(e[t] * vals[t][c] for t in range(len(keys))) / den for c in range(d)]
    return out, zm + math.log(den)


def rng_fp16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


# --------------------------------------------------------------------------- pins
def pin_scale_exhaustive(orc) -> None:
    """Every finite non-negative fp16 max maps to the correctly rounded fp32 of m/127."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)       # +0 .. largest finite
    ms = bits.view(np.float16)
    for m in ms:
        got = float(orc.block_scale(np.array([[m, -m * np.float16(0.5)]], dtype=np.float16)))
        want = fp32_nearest(Fraction(float(m)) / 127)
        assert got == want, f"scale of m={float(m)!r}: {got!r} != {want!r}"


def pin_codes_exact(orc, rng) -> None:
    """Codes equal rint-half-even of the correctly rounded fp32 quotient, over many fp16 inputs."""
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    for m in (np.float16(127.0), np.float16(65504.0), np.float16(1.0), np.float16(6.1035e-05),
              np.float16(2.0 ** -24 * 37), np.float16(3.1416), np.float16(40.72)):
        cand = finite[finite.astype(np.float64) <= float(m)]
        pick = cand[:: max(1, len(cand) // 4000)]
        xs = np.concatenate([pick, -pick, np.array([m, -m], dtype=np.float16)])
        tile = xs.reshape(1, -1)
        s = orc.block_scale(tile)
        assert float(s) == fp32_nearest(Fraction(float(m)) / 127)
        got = orc.quantize_codes(tile, s).ravel()
        want = np.array([exact_code(float(x), float(s)) for x in xs], dtype=np.int64)
        bad = np.nonzero(got.astype(np.int64) != want)[0]
        assert bad.size == 0, f"m={float(m)}: code mismatch at x={xs[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"
    # a random tile with large dynamic range
    t = rng_fp16(rng, (64, 16), 3.0)
    t[5, 7] = np.float16(-250.0)
    s = orc.block_scale(t)
    got = orc.quantize_codes(t, s)
    want = np.array([[exact_code(float(x), float(s)) for x in row] for row in t])
    assert np.array_equal(got.astype(np.int64), want)


def pin_fp32_quotient_cases(orc, rng) -> None:
    """Inputs where rounding the fp32 quotient and rounding the exact quotient disagree.

    The reading fixes the quotient x / s as an IEEE fp32 division; these rare
    cases (a few per 10^5) are found by a plain search and then checked
    against exact rational arithmetic.
    """
    pos = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)
    found = 0
    for m in rng.choice(pos[pos.astype(np.float64) > 1e-3], 48, replace=False):
        s = fp32_nearest(Fraction(float(m)) / 127)
        xs = pos[pos.astype(np.float64) <= float(m)]
        xs = np.concatenate([xs, -xs])
        q64 = xs.astype(np.float64) / s
        q32 = q64.astype(np.float32).astype(np.float64)
        cand = xs[np.rint(q64) != np.rint(q32)]
        if cand.size == 0:
            continue
        tile = np.concatenate([np.array([m], np.float16), cand]).reshape(1, -1)
        so = orc.block_scale(tile)
        assert float(so) == s
        got = orc.quantize_codes(tile, so).ravel()[1:]
        want = [exact_code(float(x), s) for x in cand]
        assert got.astype(np.int64).tolist() == want, (float(m), cand[:4], got[:4], want[:4])
        found += cand.size
    assert found >= 10, found


def pin_rounding_golden(orc) -> None:
    g = json.load(open(os.path.join(GOLDEN, "rounding_ties.json")))
    tile = np.array([g["tile"]], dtype=np.float16)
    s = orc.block_scale(tile)
    assert float(s) == g["scale"]
    assert orc.quantize_codes(tile, s).ravel().tolist() == g["codes"]


def pin_code_invariants(orc, rng) -> None:
    """|q| <= 127, the max element maps to +-127, |x - q s| <= s (1/2 + 2^-18), x_hat exact."""
    for trial in range(20):
        t = rng_fp16(rng, (int(rng.integers(1, 65)), 32), float(rng.choice([1e-3, 1.0, 10.0, 300.0])))
        s = orc.block_scale(t)
        q = orc.quantize_codes(t, s).astype(np.int64)
        assert np.all(np.abs(q) <= 127)
        i = np.unravel_index(np.argmax(np.abs(t.astype(np.float64))), t.shape)
        assert abs(q[i]) == 127
        x = t.astype(np.float64)
        err = np.abs(x - q * float(s))
        assert np.all(err <= float(s) * (0.5 + 2.0 ** -18)), err.max() / float(s)
        xh = orc.dequantize(q.astype(np.int8), s)
        for a, b in zip(xh.ravel()[:50], q.ravel()[:50]):
            assert Fraction(a) == Fraction(int(b)) * Fraction(float(s))
    z = np.zeros((7, 5), dtype=np.float16)
    assert float(orc.block_scale(z)) == 0.0 and not orc.quantize_codes(z, orc.block_scale(z)).any()


def pin_header_golden(orc) -> None:
    g = json.load(open(os.path.join(GOLDEN, "header_sizing.json")))
    for c in g["cases"]:
        n_blk, nbytes = orc.header_table_bytes(c["total_tokens"], g["hot_tokens"], c["block_size"])
        assert (n_blk, nbytes) == (c["num_blocks"], c["bytes"]), (c, n_blk, nbytes)


def _sdpa(q64, keys_by_h, vals_by_h, g):
    import torch
    import torch.nn.functional as F
    outs = []
    for hq in range(q64.shape[0]):
        h = hq // g
        qq = torch.tensor(q64[hq], dtype=torch.float64).view(1, 1, 1, -1)
        kk = torch.tensor(np.asarray(keys_by_h[h]), dtype=torch.float64).view(1, 1, len(keys_by_h[h]), -1)
        vv = torch.tensor(np.asarray(vals_by_h[h]), dtype=torch.float64).view(1, 1, len(vals_by_h[h]), -1)
        outs.append(F.scaled_dot_product_attention(qq, kk, vv).view(-1).numpy())
    return np.stack(outs)


def pin_all_hot_sdpa(orc, rng) -> None:
    """n <= hot_tokens: the cache is exact fp16, so decode is plain softmax attention (torch SDPA)."""
    for n, n_kv, g, d in ((1, 1, 1, 8), (17, 2, 2, 16), (32, 2, 4, 64), (32, 4, 1, 128)):
        k = rng_fp16(rng, (n, n_kv, d))
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, 32, 64)
        assert st.n_blocks == 0
        out, _ = orc.decode(q, st)
        keys = [k[:, h, :].astype(np.float64) for h in range(n_kv)]
        vals = [v[:, h, :].astype(np.float64) for h in range(n_kv)]
        ref = _sdpa(q.astype(np.float64), keys, vals, g)
        assert np.max(np.abs(out - ref)) < 1e-12


def pin_cold_sdpa(orc, rng) -> None:
    """With cold blocks: decode equals SDPA over (exactly re-quantised cold rows, fp16 most recent rows)."""
    for n, n_kv, g, d, hot, blk in ((100, 2, 2, 8, 32, 64), (200, 1, 4, 16, 32, 64), (75, 2, 1, 8, 16, 8)):
        k = rng_fp16(rng, (n, n_kv, d), 2.0)
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, hot, blk)
        out, lse = orc.decode(q, st)
        keys, vals = zip(*[brute_history_kv(k, v, hot, blk, h) for h in range(n_kv)])
        ref = _sdpa(q.astype(np.float64), keys, vals, g)
        assert np.max(np.abs(out - ref)) < 1e-12, np.max(np.abs(out - ref))
        for hq in range(n_kv * g):
            _, l_ref = brute_attend([float(x) for x in q[hq]], keys[hq // g], vals[hq // g])
            assert abs(lse[hq] - l_ref) < 1e-9


def pin_brute_force_decode(orc, rng) -> None:
    """Explicit loops on tiny shapes: quantise, assemble and attend with no array code at all."""
    for n, n_kv, g, d in ((70, 1, 2, 4), (130, 2, 2, 6), (33, 1, 1, 3)):
        k = rng_fp16(rng, (n, n_kv, d), 1.5)
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, 32, 64)
        out, lse = orc.decode(q, st)
        for hq in range(n_kv * g):
            keys, vals = brute_history_kv(k, v, 32, 64, hq // g)
            o_ref, l_ref = brute_attend([float(x) for x in q[hq]], keys, vals)
            assert max(abs(a - b) for a, b in zip(out[hq], o_ref)) < 1e-12
            assert abs(lse[hq] - l_ref) < 1e-12


def pin_convexity(orc, rng) -> None:
    """Outputs are convex combinations of attended value rows; equal logits give the mean row."""
    n, n_kv, g, d = 300, 2, 2, 16
    k = rng_fp16(rng, (n, n_kv, d))
    v = rng_fp16(rng, (n, n_kv, d), 3.0)
    q = rng_fp16(rng, (n_kv * g, d))
    st = orc.build_state(k, v, 32, 64)
    out, _ = orc.decode(q, st)
    for hq in range(n_kv * g):
        _, vals = brute_history_kv(k, v, 32, 64, hq // g)
        vv = np.asarray(vals)
        assert np.all(out[hq] >= vv.min(axis=0) - 1e-12) and np.all(out[hq] <= vv.max(axis=0) + 1e-12)
    # zero query: every logit is 0, so the output is the plain mean of the attended value rows
    out0, lse0 = orc.decode(np.zeros_like(q), st)
    for hq in range(n_kv * g):
        _, vals = brute_history_kv(k, v, 32, 64, hq // g)
        assert np.max(np.abs(out0[hq] - np.mean(np.asarray(vals), axis=0))) < 1e-12
        assert abs(lse0[hq] - math.log(n)) < 1e-12


def pin_hot_is_most_recent(orc, rng) -> None:
    """The FP16 rows must be the most recent ones: a distinct last token must come back exactly."""
    n, d = 96, 8
    k = np.zeros((n, 1, d), dtype=np.float16)
    v = np.zeros((n, 1, d), dtype=np.float16)
    v[:, 0, :] = np.float16(1.0)
    k[-1, 0, 0] = np.float16(64.0)              # the newest token dominates the softmax
    v[-1, 0, :] = np.float16(0.1)               # 0.1 is not a multiple of any int8 scale of this tile
    q = np.zeros((1, d), dtype=np.float16)
    q[0, 0] = np.float16(8.0)
    st = orc.build_state(k, v, 32, 64)
    out, _ = orc.decode(q, st)
    # softmax weight of every other token is exp(-64*8/sqrt(8)) < 1e-78, so out is v[-1] in fp16 exactly
    assert np.all(out[0] == float(np.float16(0.1)))


def brute_topk(q, k_hist, hot, blk, n_kv, g, kk, bits=8):
    """Loops: dequantised cold keys, mean cosine over the group, softmax per block, sort with tie rule."""
    n = len(k_hist)
    n_cold = n - min(n, hot)
    result = []
    for h in range(n_kv):
        keys, _ = brute_history_kv(k_hist, k_hist, hot, blk, h, bits)
        keys = keys[:n_cold]
        c = []
        for t in range(n_cold):
            acc = 0.0
            kn = math.sqrt(sum(x * x for x in keys[t]))
            for hq in range(h * g, (h + 1) * g):
                qr = [float(x) for x in q[hq]]
                qn = math.sqrt(sum(x * x for x in qr))
                acc += 0.0 if kn == 0 or qn == 0 else sum(a * b for a, b in zip(qr, keys[t])) / (qn * kn)
            c.append(acc / g)
        p = [0.0] * n_cold
        for j0 in range(0, n_cold, blk):
            w = list(range(j0, min(j0 + blk, n_cold)))
            mx = max(c[t] for t in w)
            den = sum(math.exp(c[t] - mx) for t in w)
            for t in w:
                p[t] = math.exp(c[t] - mx) / den
        order = sorted(range(n_cold), key=lambda t: (-p[t], t))
        chosen = sorted(order[:kk])
        result.append((chosen + [-1] * kk)[:kk])
    return np.array(result)


def pin_topk_brute(orc, rng) -> None:
    for n, n_kv, g, d, kk in ((200, 2, 2, 8, 20), (150, 1, 4, 8, 200), (97, 2, 1, 4, 7)):
        k = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, k, 32, 64)
        idx, p, _ = orc.topk_select(q, st, kk)
        assert np.array_equal(idx, brute_topk(q, k, 32, 64, n_kv, g, kk))
        for j in range(st.n_blocks):   # each window is a probability distribution
            lo = j * 64
            assert np.allclose(p[:, lo:lo + int(st.n_valid[j])].sum(axis=1), 1.0, atol=1e-12)


def pin_topk_ties_lower_index(orc) -> None:
    """Identical keys tie exactly; the lower token index must win."""
    n, d = 32 + 128, 4
    k = np.ones((n, 1, d), dtype=np.float16)
    q = np.ones((1, d), dtype=np.float16)
    st = orc.build_state(k, k, 32, 64)
    idx, _, _ = orc.topk_select(q, st, 5)
    assert idx[0].tolist() == [0, 1, 2, 3, 4]
    # one weaker token in window 1 lifts its 63 neighbours above window 0's uniform 1/64,
    # so the three lowest indices of window 1 other than the weak token win
    k2 = k.copy()
    k2[70, 0, :] = np.array([1, 1, 1, -1], dtype=np.float16)
    st2 = orc.build_state(k2, k2, 32, 64)
    idx2, p2, _ = orc.topk_select(q, st2, 3)
    assert idx2[0].tolist() == [64, 65, 66]
    assert p2[0, 0] == 1.0 / 64
    assert abs(p2[0, 64] - 1.0 / (63 + math.exp(-0.5))) < 1e-15


def pin_topk_scale_invariance(orc, rng) -> None:
    """cos(q, s*code) == cos(q, code): scoring codes equals scoring dequantised keys."""
    n, n_kv, g, d = 32 + 3 * 64, 2, 2, 16
    k = rng_fp16(rng, (n, n_kv, d), 5.0)
    q = rng_fp16(rng, (n_kv * g, d))
    st = orc.build_state(k, k, 32, 64)
    c = orc.token_scores(q, st)
    for h in range(n_kv):
        for t in range(0, st.n_cold, 17):
            j, r = divmod(t, 64)
            code = st.codes[j, h, 0, r].astype(np.float64)
            want = np.mean([float(q[hq].astype(np.float64) @ code) /
                            (np.linalg.norm(q[hq].astype(np.float64)) * np.linalg.norm(code))
                            for hq in range(h * g, (h + 1) * g)])
            assert abs(c[h, t] - want) < 1e-12


def pin_topk_all_selected(orc, rng) -> None:
    """K >= cold tokens: everything is selected and sparse decode equals dense decode."""
    n, n_kv, g, d = 32 + 100, 2, 2, 8
    k = rng_fp16(rng, (n, n_kv, d))
    v = rng_fp16(rng, (n, n_kv, d))
    q = rng_fp16(rng, (n_kv * g, d))
    st = orc.build_state(k, v, 32, 64)
    idx, _, _ = orc.topk_select(q, st, 128)
    assert idx[:, :100].tolist() == [list(range(100))] * n_kv and np.all(idx[:, 100:] == -1)
    o1, l1 = orc.sparse_decode(q, st, idx)
    o2, l2 = orc.decode(q, st)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def pin_sparse_subset(orc, rng) -> None:
    """Sparse decode equals SDPA over hot rows plus exactly the selected cold rows."""
    n, n_kv, g, d = 32 + 3 * 64 + 10, 2, 2, 8
    k = rng_fp16(rng, (n, n_kv, d))
    v = rng_fp16(rng, (n, n_kv, d))
    q = rng_fp16(rng, (n_kv * g, d))
    st = orc.build_state(k, v, 32, 64)
    idx = np.full((n_kv, 16), -1)
    idx[0, :5] = [0, 3, 64, 150, 201]
    idx[1, :3] = [10, 11, 199]
    out, _ = orc.sparse_decode(q, st, idx)
    keys_sel, vals_sel = [], []
    for h in range(n_kv):
        keys, vals = brute_history_kv(k, v, 32, 64, h)
        n_cold = n - 32
        sel = [int(t) for t in idx[h] if t >= 0]
        keys_sel.append([keys[t] for t in sel] + keys[n_cold:])
        vals_sel.append([vals[t] for t in sel] + vals[n_cold:])
    ref = _sdpa(q.astype(np.float64), keys_sel, vals_sel, g)
    assert np.max(np.abs(out - ref)) < 1e-12


# --------------------------------------------------------------------------- INT4 and FP16 cold zones
def pin_int4_scale_exhaustive(orc) -> None:
    """Every finite non-negative fp16 max maps to the correctly rounded fp32 of m/7 at 4 bits."""
    ms = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    for m in ms:
        got = float(orc.block_scale(np.array([[m, -m * np.float16(0.25)]], dtype=np.float16), 4))
        want = fp32_nearest(Fraction(float(m)) / 7)
        assert got == want, f"4-bit scale of m={float(m)!r}: {got!r} != {want!r}"


def pin_int4_codes_exact(orc, rng) -> None:
    """4-bit codes equal rint-half-even of the correctly rounded fp32 quotient, clipped to +-7, for every
    fp16 input below a set of maxima (and the inputs next to each rounding boundary k + 1/2)."""
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    for m in (np.float16(7.0), np.float16(65504.0), np.float16(1.0), np.float16(6.1035e-05),
              np.float16(2.0 ** -24 * 37), np.float16(3.1416), np.float16(40.72), np.float16(0.3)):
        cand = finite[finite.astype(np.float64) <= float(m)]
        pick = cand[:: max(1, len(cand) // 3000)]
        s = fp32_nearest(Fraction(float(m)) / 7)
        near = []
        for k in range(7):
            t = np.float16((k + 0.5) * s)
            near += [np.nextafter(t, np.float16(-np.inf)), t, np.nextafter(t, np.float16(np.inf))]
        near = np.array([x for x in near if 0 < float(x) <= float(m)], dtype=np.float16)
        xs = np.concatenate([pick, -pick, near, -near, np.array([m, -m], dtype=np.float16)])
        tile = xs.reshape(1, -1)
        so = orc.block_scale(tile, 4)
        assert float(so) == s
        got = orc.quantize_codes(tile, so, 4).ravel()
        want = np.array([exact_code(float(x), s, 7) for x in xs], dtype=np.int64)
        bad = np.nonzero(got.astype(np.int64) != want)[0]
        assert bad.size == 0, f"m={float(m)}: 4-bit code mismatch at x={xs[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"


def pin_int4_code_invariants(orc, rng) -> None:
    """|q| <= 7, the max element maps to +-7, |x - q s| <= s (1/2 + 2^-18), x_hat = q s exactly."""
    for trial in range(20):
        t = rng_fp16(rng, (int(rng.integers(1, 65)), 32), float(rng.choice([1e-3, 1.0, 10.0, 300.0])))
        s = orc.block_scale(t, 4)
        q = orc.quantize_codes(t, s, 4).astype(np.int64)
        assert np.all(np.abs(q) <= 7)
        i = np.unravel_index(np.argmax(np.abs(t.astype(np.float64))), t.shape)
        assert abs(q[i]) == 7
        err = np.abs(t.astype(np.float64) - q * float(s))
        assert np.all(err <= float(s) * (0.5 + 2.0 ** -18))
        xh = orc.dequantize(q.astype(np.int8), s)
        for a, b in zip(xh.ravel()[:50], q.ravel()[:50]):
            assert Fraction(a) == Fraction(int(b)) * Fraction(float(s))


def pin_int4_cold_sdpa(orc, rng) -> None:
    """4-bit cold blocks: decode equals SDPA over exactly re-quantised (limit 7) cold rows + fp16 hot rows,
    and explicit loops agree on a tiny shape."""
    for n, n_kv, g, d, hot, blk in ((100, 2, 2, 8, 32, 64), (200, 1, 4, 16, 32, 64), (75, 2, 1, 8, 16, 8)):
        k = rng_fp16(rng, (n, n_kv, d), 2.0)
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, hot, blk, 4)
        out, lse = orc.decode(q, st)
        keys, vals = zip(*[brute_history_kv(k, v, hot, blk, h, 4) for h in range(n_kv)])
        ref = _sdpa(q.astype(np.float64), keys, vals, g)
        assert np.max(np.abs(out - ref)) < 1e-12, np.max(np.abs(out - ref))
    n, n_kv, g, d = 90, 1, 2, 4
    k = rng_fp16(rng, (n, n_kv, d), 1.5)
    v = rng_fp16(rng, (n, n_kv, d))
    q = rng_fp16(rng, (n_kv * g, d))
    st = orc.build_state(k, v, 32, 64, 4)
    out, lse = orc.decode(q, st)
    for hq in range(n_kv * g):
        keys, vals = brute_history_kv(k, v, 32, 64, hq // g, 4)
        o_ref, l_ref = brute_attend([float(x) for x in q[hq]], keys, vals)
        assert max(abs(a - b) for a, b in zip(out[hq], o_ref)) < 1e-12
        assert abs(lse[hq] - l_ref) < 1e-12


def pin_fp16_cold_is_dense_attention(orc, rng) -> None:
    """quantization_bits 0: the cold zone keeps the fp16 values, so decode over any history (cold blocks
    included) equals plain softmax attention over the whole fp16 history (torch SDPA), and the state
    holds the history rows with scale 1."""
    for n, n_kv, g, d in ((300, 2, 2, 16), (32 + 64 * 3 + 5, 1, 4, 8), (33, 2, 1, 8)):
        k = rng_fp16(rng, (n, n_kv, d), 40.0)
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, 32, 64, 0)
        out, lse = orc.decode(q, st)
        keys = [k[:, h, :].astype(np.float64) for h in range(n_kv)]
        vals = [v[:, h, :].astype(np.float64) for h in range(n_kv)]
        ref = _sdpa(q.astype(np.float64), keys, vals, g)
        assert np.max(np.abs(out - ref)) < 1e-12
        n_cold = n - min(n, 32)
        for j in range(st.n_blocks):
            nv = int(st.n_valid[j])
            rows = k[j * 64:j * 64 + nv].transpose(1, 0, 2)
            assert np.array_equal(st.codes[j, :, 0, :nv].view(np.uint16), rows.view(np.uint16))
            assert np.all(st.scales[j] == 1.0)
        assert st.n_cold == n_cold


def pin_topk_other_widths(orc, rng) -> None:
    """Top-K over 4-bit cold blocks (cosine of the codes) and over an FP16 cold zone (cosine of the fp16
    keys) against the brute-force loops."""
    for bits in (4, 0):
        n, n_kv, g, d, kk = 200, 2, 2, 8, 20
        k = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, k, 32, 64, bits)
        idx, _, _ = orc.topk_select(q, st, kk)
        assert np.array_equal(idx, brute_topk(q, k, 32, 64, n_kv, g, kk, bits)), bits


# --------------------------------------------------------------------------- debug statistics
def pin_quant_error_exact(orc, rng) -> None:
    """The largest |x - q s| of each tile against exact rational arithmetic (codes and scales from the
    exact helpers), for 8 and 4 bits; rounding bounds it by s/2; FP16 tiles and tiles of exact
    multiples of the scale have error 0."""
    for bits, lim in ((8, 127), (4, 7)):
        n, n_kv, d = 32 + 2 * 64 + 9, 2, 8
        k = rng_fp16(rng, (n, n_kv, d), 3.0)
        v = rng_fp16(rng, (n, n_kv, d))
        err = orc.quant_errors(k, v, 32, 64, bits)
        n_cold = n - 32
        for j in range(err.shape[0]):
            rows = range(j * 64, min((j + 1) * 64, n_cold))
            for h in range(n_kv):
                for c, src in enumerate((k, v)):
                    tile = np.array([src[t][h] for t in rows], dtype=np.float16)
                    s = exact_scale(tile, lim)
                    want = max(abs(Fraction(float(x)) - exact_code(float(x), s, lim) * Fraction(s)) for x in tile.ravel())
                    assert Fraction(err[j, h, c]) == want, (bits, j, h, c)
                    assert err[j, h, c] <= s / 2 * (1 + 2.0 ** -17)
    ints = np.tile(np.arange(-63, 64, dtype=np.float16)[:, None, None], (1, 1, 4))[:96]
    ints[0, 0, 0] = ints[64, 0, 0] = np.float16(127.0)   # each block's max is 127: s = 1, every value a multiple
    hist = np.concatenate([ints, rng_fp16(rng, (32, 1, 4))])
    assert np.all(orc.quant_errors(hist, hist, 32, 64, 8)[:, :, 0] == 0.0)
    assert np.all(orc.quant_errors(hist, hist, 32, 64, 0) == 0.0)


def pin_entropy(orc, rng) -> None:
    """Entropy of the decode softmax: equal logits give ln n (zero query); one overwhelming token gives
    ~0; explicit loops agree on a tiny shape; the sparse form covers exactly the selected tokens."""
    n, n_kv, g, d = 200, 2, 2, 8
    k = rng_fp16(rng, (n, n_kv, d))
    v = rng_fp16(rng, (n, n_kv, d))
    st = orc.build_state(k, v, 32, 64)
    ent0 = orc.attention_entropy(np.zeros((n_kv * g, d), np.float16), st)
    assert np.all(np.abs(ent0 - math.log(n)) < 1e-12)
    kk = np.zeros((96, 1, d), dtype=np.float16)
    kk[-1, 0, 0] = np.float16(64.0)
    q1 = np.zeros((1, d), dtype=np.float16)
    q1[0, 0] = np.float16(8.0)
    assert orc.attention_entropy(q1, orc.build_state(kk, kk, 32, 64))[0] < 1e-60
    q = rng_fp16(rng, (n_kv * g, d))
    ent = orc.attention_entropy(q, st)
    for hq in range(n_kv * g):
        keys, _ = brute_history_kv(k, v, 32, 64, hq // g)
        z = [sum(float(q[hq][c]) * kr[c] for c in range(d)) / math.sqrt(d) for kr in keys]
        zm = max(z)
        e = [math.exp(x - zm) for x in z]
        tot = sum(e)
        want = -sum((x / tot) * math.log(x / tot) for x in e if x > 0)
        assert abs(ent[hq] - want) < 1e-12
    idx = np.full((n_kv, 8), -1)
    idx[0, :3] = [0, 5, 100]
    idx[1, :2] = [7, 150]
    ent_s = orc.attention_entropy(q, st, idx)
    for hq in range(n_kv * g):
        h = hq // g
        keys, _ = brute_history_kv(k, v, 32, 64, h)
        sel = [int(t) for t in idx[h] if t >= 0] + list(range(n - 32, n))
        z = [sum(float(q[hq][c]) * keys[t][c] for c in range(d)) / math.sqrt(d) for t in sel]
        zm = max(z)
        e = [math.exp(x - zm) for x in z]
        tot = sum(e)
        want = -sum((x / tot) * math.log(x / tot) for x in e if x > 0)
        assert abs(ent_s[hq] - want) < 1e-12


# --------------------------------------------------------------------------- compacted sparse store
def pin_sparse_store(orc, rng) -> None:
    """The store holds exactly the selected rows (explicit loops over blocks and rows), in selection
    order, with each row's own block scales; masked and out-of-range entries are skipped, duplicates
    kept; decoding over it equals the sparse decode and SDPA over the selected dequantised rows."""
    for bits in (8, 4, 0):
        n, n_kv, g, d = 32 + 3 * 64 + 10, 2, 2, 8
        k = rng_fp16(rng, (n, n_kv, d))
        v = rng_fp16(rng, (n, n_kv, d))
        q = rng_fp16(rng, (n_kv * g, d))
        st = orc.build_state(k, v, 32, 64, bits)
        n_cold = n - 32
        idx = np.full((n_kv, 12), -1)
        idx[0, :7] = [0, 3, 64, 150, 201, 3, n_cold + 5]     # a duplicate and an out-of-range entry
        idx[1, :4] = [10, 11, 199, 63]
        store = orc.sparse_store(st, idx)
        keys, vals = zip(*[brute_history_kv(k, v, 32, 64, h, bits) for h in range(n_kv)])
        want_rows = [[0, 3, 64, 150, 201, 3], [10, 11, 199, 63]]
        assert store.counts.tolist() == [6, 4]
        for h in range(n_kv):
            for i, t in enumerate(want_rows[h]):
                xk = store.k_codes[h][i].astype(np.float64) * float(store.k_scales[h][i])
                xv = store.v_codes[h][i].astype(np.float64) * float(store.v_scales[h][i])
                assert np.array_equal(xk, np.array(keys[h][t])) and np.array_equal(xv, np.array(vals[h][t]))
        empty = orc.sparse_store(st, np.full((n_kv, 4), -1))  # a selection with no valid entry
        assert empty.counts.tolist() == [0] * n_kv and all(x.shape == (0, d) for x in empty.k_codes)
        o1, l1 = orc.decode_over_store(q, st, store)
        o2, l2 = orc.sparse_decode(q, st, np.where((idx >= 0) & (idx < n_cold), idx, -1))
        assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
        sel_k = [[keys[h][t] for t in want_rows[h]] + keys[h][n_cold:] for h in range(n_kv)]
        sel_v = [[vals[h][t] for t in want_rows[h]] + vals[h][n_cold:] for h in range(n_kv)]
        ref = _sdpa(q.astype(np.float64), sel_k, sel_v, g)
        assert np.max(np.abs(o1 - ref)) < 1e-12


ALL_PINS = [
    ("scale_exhaustive", lambda o, r: pin_scale_exhaustive(o)),
    ("codes_exact", pin_codes_exact),
    ("fp32_quotient_cases", pin_fp32_quotient_cases),
    ("rounding_golden", lambda o, r: pin_rounding_golden(o)),
    ("code_invariants", pin_code_invariants),
    ("header_golden", lambda o, r: pin_header_golden(o)),
    ("all_hot_sdpa", pin_all_hot_sdpa),
    ("cold_sdpa", pin_cold_sdpa),
    ("brute_force_decode", pin_brute_force_decode),
    ("convexity", pin_convexity),
    ("hot_is_most_recent", pin_hot_is_most_recent),
    ("topk_brute", pin_topk_brute),
    ("topk_ties_lower_index", lambda o, r: pin_topk_ties_lower_index(o)),
    ("topk_scale_invariance", pin_topk_scale_invariance),
    ("topk_all_selected", pin_topk_all_selected),
    ("sparse_subset", pin_sparse_subset),
    ("int4_scale_exhaustive", lambda o, r: pin_int4_scale_exhaustive(o)),
    ("int4_codes_exact", pin_int4_codes_exact),
    ("int4_code_invariants", pin_int4_code_invariants),
    ("int4_cold_sdpa", pin_int4_cold_sdpa),
    ("fp16_cold_is_dense_attention", pin_fp16_cold_is_dense_attention),
    ("topk_other_widths", pin_topk_other_widths),
    ("quant_error_exact", pin_quant_error_exact),
    ("entropy", pin_entropy),
    ("sparse_store", pin_sparse_store),
]
