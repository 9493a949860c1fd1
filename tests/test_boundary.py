"""CPU: the C-ABI library loads, exports every declared entry point, and rejects
bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
hkv = pytest.importorskip("int8_kv_cache_hkv_amd")

INVALID, UNSUPPORTED, NULLP, CAPACITY, WORKSPACE, ALIGN = -1, -2, -3, -4, -5, -7


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hkv.h")).read()
    return sorted(set(re.findall(r"^(?:hkv_status|const char\*)\s+(hkv_\w+)\(", src, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("hkv_create", "hkv_append", "hkv_decode_attn", "hkv_topk_select", "hkv_destroy"):
        assert must in names
    assert sorted(hkv.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hkv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _create(*args):
    h = ctypes.c_void_p()
    st = hkv._lib.hkv_create(*args, ctypes.byref(h))
    if st == 0:
        hkv._lib.hkv_destroy(h)
    return st


@pytest.mark.parametrize("hot,block,bits,want", [
    (32, 64, 8, 0), (16, 64, 8, 0), (64, 64, 8, 0), (128, 64, 8, 0),
    (33, 64, 8, INVALID), (48, 64, 8, INVALID), (8, 64, 8, INVALID), (256, 64, 8, INVALID),
    (32, 63, 8, INVALID), (32, 0, 8, INVALID), (32, -8, 8, INVALID),
    (32, 64, 7, INVALID), (32, 64, 16, INVALID),
    (32, 64, 4, UNSUPPORTED), (32, 64, 0, UNSUPPORTED), (32, 128, 8, UNSUPPORTED), (32, 32, 8, UNSUPPORTED),
])
def test_create_protocol_rules(hot, block, bits, want):
    assert _create(8, 128, hot, block, bits) == want


def test_create_shapes():
    assert _create(8, 64, 32, 64, 8) == 0
    assert _create(8, 96, 32, 64, 8) == UNSUPPORTED
    assert _create(0, 128, 32, 64, 8) == INVALID
    assert hkv._lib.hkv_create(8, 128, 32, 64, 8, None) == NULLP


def test_header_sizing_worked_example():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "header_sizing.json")))
    for c in g["cases"]:
        nb, by = hkv.hkv_header_table_bytes(g["hot_tokens"], c["block_size"], c["total_tokens"])
        assert (nb, by) == (c["num_blocks"], c["bytes"])
    with pytest.raises(hkv.HKVError):
        hkv.hkv_header_table_bytes(48, 64, 1000)


def test_cache_sizes():
    h = hkv.hkv_create(8, 128)
    try:
        s = hkv.hkv_cache_sizes(h, 8, 2048)
        assert s.max_blocks_per_seq == 32 and s.num_phys_blocks == 256
        assert s.hot == 8 * 8 * 32 * 2 * 128 * 2
        assert s.tail == 8 * 8 * 2 * 64 * 128 * 2
        assert s.cold == 256 * 8 * 2 * 64 * 128
        assert s.scales == 256 * 8 * 2 * 4
        assert s.headers == 8 * 32 * 16
        s2 = hkv.hkv_cache_sizes(h, 2, 32)          # all-hot capacity: no cold blocks
        assert s2.max_blocks_per_seq == 0 and s2.cold == 0
        s3 = hkv.hkv_cache_sizes(h, 4, 131072, 10000)
        assert s3.max_blocks_per_seq == 2048 and s3.num_phys_blocks == 10000
        with pytest.raises(hkv.HKVError):
            hkv.hkv_cache_sizes(h, 0, 10)
    finally:
        hkv.hkv_destroy(h)


class FakeCache:
    """Descriptor over fake (never dereferenced) aligned addresses, for host-side error paths."""

    def __init__(self, h, batch=2, max_blocks=4, lens=(0, 0)):
        self.h = h
        self.lens = np.array(lens, dtype=np.int32)
        base = 1 << 40
        self.desc = hkv.CacheDesc(batch, max_blocks, batch * max_blocks, base, base + 4096, base + 8192,
                                  base + 12288, base + 16384, base + 20480, self.lens.ctypes.data)


def test_workspace_bytes():
    h = hkv.hkv_create(8, 128)
    try:
        fc = FakeCache(h, batch=8, max_blocks=32, lens=[0] * 8)
        a = hkv.hkv_workspace_bytes(h, fc.desc, 32)
        b = hkv.hkv_workspace_bytes(h, fc.desc, 32, 512)
        assert a >= 8 * 8 * 4 * 130 * 4 and b >= max(a, 8 * 8 * 32 * 64 * 4)
        for nq, k in ((30, 0), (0, 0), (32, 513), (32, -1)):
            with pytest.raises(hkv.HKVError):
                hkv.hkv_workspace_bytes(h, fc.desc, nq, k)
    finally:
        hkv.hkv_destroy(h)


def _status(fn, *args):
    return fn(*args)


def test_append_host_errors():
    h = hkv.hkv_create(8, 128)
    lib = hkv._lib
    try:
        fc = FakeCache(h, batch=2, max_blocks=4, lens=[0, 0])
        d = ctypes.byref(fc.desc)
        fake_k = (1 << 41)
        n_ok = np.array([1, 1], np.int32)
        # capacity: 4 blocks of 64 + 32 hot = 288 tokens per sequence
        n_big = np.array([289, 0], np.int32)
        assert lib.hkv_append(h, d, fake_k, fake_k, n_big.ctypes.data, 289, None) == CAPACITY
        n_neg = np.array([-1, 0], np.int32)
        assert lib.hkv_append(h, d, fake_k, fake_k, n_neg.ctypes.data, 1, None) == INVALID
        assert lib.hkv_append(h, d, fake_k, fake_k, n_ok.ctypes.data, 0, None) == INVALID   # count > max_n_new
        assert lib.hkv_append(h, d, fake_k, fake_k, None, 1, None) == NULLP
        assert lib.hkv_append(h, d, None, None, n_ok.ctypes.data, 1, None) == NULLP
        assert lib.hkv_append(h, d, fake_k + 2, fake_k, n_ok.ctypes.data, 1, None) == ALIGN
        zero = np.zeros(2, np.int32)
        assert lib.hkv_append(h, d, None, None, zero.ctypes.data, 0, None) == 0      # nothing to do
        fc.desc.hot += 256
        assert lib.hkv_append(h, d, fake_k, fake_k, n_ok.ctypes.data, 1, None) == ALIGN
        assert fc.lens.tolist() == [0, 0]   # the mirror is untouched on error
    finally:
        hkv.hkv_destroy(h)


def test_decode_and_topk_host_errors():
    h = hkv.hkv_create(8, 128)
    lib = hkv._lib
    try:
        fc = FakeCache(h, batch=2, max_blocks=4, lens=[0, 5])
        d = ctypes.byref(fc.desc)
        q = out = ws = (1 << 41)
        big = 1 << 30
        assert lib.hkv_decode_attn(h, d, q, 32, None, 0, out, None, ws, big, None) == INVALID   # empty sequence
        fc.lens[0] = 3
        assert lib.hkv_decode_attn(h, d, q, 30, None, 0, out, None, ws, big, None) == INVALID   # 30 % 8
        assert lib.hkv_decode_attn(h, d, q, 24, None, 0, out, None, ws, big, None) == UNSUPPORTED  # G = 3
        assert lib.hkv_decode_attn(h, d, q, 32, q, 0, out, None, ws, big, None) == INVALID     # k_sel 0
        assert lib.hkv_decode_attn(h, d, q, 32, q, 513, out, None, ws, big, None) == INVALID
        assert lib.hkv_decode_attn(h, d, q, 32, None, 0, out, None, ws, 16, None) == WORKSPACE
        assert lib.hkv_decode_attn(h, d, q, 32, None, 0, out, None, None, big, None) == WORKSPACE
        assert lib.hkv_decode_attn(h, d, None, 32, None, 0, out, None, ws, big, None) == NULLP
        ad = lib.hkv_append_decode
        assert ad(h, d, q, q, q, 30, out, None, ws, big, None) == INVALID        # 30 % 8
        assert ad(h, d, q, q, q, 24, out, None, ws, big, None) == UNSUPPORTED    # G = 3
        assert ad(h, d, None, q, q, 32, out, None, ws, big, None) == NULLP
        assert ad(h, d, q, q, None, 32, out, None, ws, big, None) == NULLP
        assert ad(h, d, q, q, q, 32, out, None, ws, 16, None) == WORKSPACE
        assert ad(h, d, q + 8, q, q, 32, out, None, ws, big, None) == ALIGN
        fc.lens[1] = 32 + 4 * 64        # full: the appended token needs a fifth cold block
        assert ad(h, d, q, q, q, 32, out, None, ws, big, None) == CAPACITY
        assert fc.lens.tolist() == [3, 32 + 4 * 64]   # the mirror is untouched on error
        fc.lens[1] = -1
        assert ad(h, d, q, q, q, 32, out, None, ws, big, None) == INVALID
        fc.lens[1] = 5
        assert lib.hkv_topk_select(h, d, q, 32, 0, out, ws, big, None) == INVALID
        assert lib.hkv_topk_select(h, d, q, 32, 513, out, ws, big, None) == INVALID
        assert lib.hkv_topk_select(h, d, q, 32, 512, out, ws, 16, None) == WORKSPACE
        assert lib.hkv_topk_select(h, d, q, 24, 16, out, ws, big, None) == UNSUPPORTED
    finally:
        hkv.hkv_destroy(h)


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert hkv.hkv_status_string(st)
    assert hkv.hkv_status_string(99) == "unknown status"
