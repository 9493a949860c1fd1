"""CPU: the oracle against its pins, and planted oracle mistakes against the pins."""
import numpy as np
import pytest

import oracle.hkv_oracle as orc
from tests import oracle_pins as pins


@pytest.mark.parametrize("name,fn", pins.ALL_PINS, ids=[n for n, _ in pins.ALL_PINS])
def test_pin(name, fn):
    fn(orc, np.random.default_rng(1234))


_LIM = {8: 127, 4: 7}


def _m_scale_128(x, bits=8):
    x = np.asarray(x)
    div = 128.0 if bits == 8 else 7.0
    return np.float32(float(np.max(np.abs(x.astype(np.float64)))) / div) if x.size else np.float32(0)


def _m_int4_scale_8(x, bits=8):
    x = np.asarray(x)
    div = 127.0 if bits == 8 else 8.0
    return np.float32(float(np.max(np.abs(x.astype(np.float64)))) / div) if x.size else np.float32(0)


def _m_round_half_up(x, s, bits=8):
    if float(s) == 0.0:
        return np.zeros(np.asarray(x).shape, np.int8)
    quot = (np.asarray(x).astype(np.float64) / np.float64(s)).astype(np.float32).astype(np.float64)
    return np.clip(np.floor(quot + 0.5), -_LIM[bits], _LIM[bits]).astype(np.int8)


def _m_no_fp32_quotient(x, s, bits=8):
    if float(s) == 0.0:
        return np.zeros(np.asarray(x).shape, np.int8)
    return np.clip(np.rint(np.asarray(x).astype(np.float64) / np.float64(s)), -_LIM[bits], _LIM[bits]).astype(np.int8)


def _m_int4_with_int8_scale(x, bits=8):
    x = np.asarray(x)
    return np.float32(float(np.max(np.abs(x.astype(np.float64)))) / 127.0) if x.size else np.float32(0)


def _m_fp16_cold_quantised(k_rows, v_rows, block_size, bits=8):
    return _REAL["quantize_block"](k_rows, v_rows, block_size, 8 if bits == 0 else bits)


def _m_split_first_hot(n, hot):
    # hot = the FIRST tokens instead of the most recent ones: split sizes are the same, so the
    # planted mistake is the position of the hot rows; emulate it by reversing the history
    return min(n, hot), n - min(n, hot)


def _mutant_build_state_first_hot(k_hist, v_hist, hot, block, quant_bits=8):
    st = _REAL["build_state"](k_hist[::-1].copy(), v_hist[::-1].copy(), hot, block, quant_bits)
    return st


def _m_attend_no_sqrt(q, keys, vals):
    z = keys @ q
    e = np.exp(z - z.max())
    return (e @ vals) / e.sum(), float(z.max() + np.log(e.sum()))


def _m_attend_sign(q, keys, vals):
    z = -(keys @ q) / np.sqrt(q.shape[0])
    e = np.exp(z - z.max())
    return (e @ vals) / e.sum(), float(z.max() + np.log(e.sum()))


def _m_window_global(c, n_valid, block):
    e = np.exp(c - c.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _m_cosine_no_knorm(q, state):
    q64 = np.asarray(q, np.float16).astype(np.float64)
    g = q64.shape[0] // state.hot_k.shape[1]
    out = np.zeros((state.hot_k.shape[1], state.n_cold))
    for h in range(out.shape[0]):
        ck, _ = orc.cold_kv(state, h)
        for hq in range(h * g, (h + 1) * g):
            out[h] += ck @ q64[hq] / np.linalg.norm(q64[hq])
        out[h] /= g
    return out


def _m_entropy_log2(q, state, sel=None):
    return _REAL["attention_entropy"](q, state, sel) / np.log(2.0)


def _m_quant_error_relative(k_hist, v_hist, hot, block, bits=8):
    st = _REAL["build_state"](k_hist, v_hist, hot, block, bits)
    err = _REAL["quant_errors"](k_hist, v_hist, hot, block, bits)
    return err / np.where(st.scales > 0, st.scales, 1.0)


def _m_store_block_scale_of_first(state, idx):
    st = _REAL["sparse_store"](state, idx)
    for h in range(len(st.k_scales)):   # every row dequantised with the first row's block scale
        if len(st.k_scales[h]):
            st.k_scales[h][:] = st.k_scales[h][0]
            st.v_scales[h][:] = st.v_scales[h][0]
    return st


_REAL = {"build_state": orc.build_state, "quantize_block": orc.quantize_block, "sparse_store": orc.sparse_store,
         "attention_entropy": orc.attention_entropy, "quant_errors": orc.quant_errors}

MUTANTS = [
    ("scale_divides_by_128", "block_scale", _m_scale_128),
    ("round_half_up", "quantize_codes", _m_round_half_up),
    ("quotient_not_rounded_to_fp32", "quantize_codes", _m_no_fp32_quotient),
    ("hot_zone_is_first_tokens", "build_state", _mutant_build_state_first_hot),
    ("logits_missing_inv_sqrt_d", "attend", _m_attend_no_sqrt),
    ("logit_sign_flipped", "attend", _m_attend_sign),
    ("softmax_over_all_tokens_not_windows", "window_softmax", _m_window_global),
    ("cosine_missing_key_norm", "token_scores", _m_cosine_no_knorm),
    ("int4_scale_divides_by_8", "block_scale", _m_int4_scale_8),
    ("int4_block_uses_the_int8_scale", "block_scale", _m_int4_with_int8_scale),
    ("fp16_cold_zone_quantised", "quantize_block", _m_fp16_cold_quantised),
    ("entropy_in_bits_not_nats", "attention_entropy", _m_entropy_log2),
    ("quant_error_relative_to_scale", "quant_errors", _m_quant_error_relative),
    ("store_rows_share_one_scale", "sparse_store", _m_store_block_scale_of_first),
]


@pytest.mark.parametrize("name,attr,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, attr, fn):
    monkeypatch.setattr(orc, attr, fn)
    caught = None
    for pin_name, pin in pins.ALL_PINS:
        try:
            pin(orc, np.random.default_rng(1234))
        except (AssertionError, ValueError, IndexError):
            caught = pin_name
            break
    assert caught, f"no pin caught the planted mistake {name}"
