"""Python binding of libhkv (hybrid FP16-hot / INT8-cold KV cache, MI355X).

Argument marshalling only: every step of the cache and attention path runs
in the HIP kernels of ``libhkv.so``.  The functions below carry the C-ABI
names (``hkv_create``, ``hkv_append``, ``hkv_decode_attn``,
``hkv_topk_select``, ...) and take torch tensors for device memory and the
current torch stream for ordering.  ``HybridKVCache`` is a convenience owner
of the cache buffers.

The library must have been built (``python -m int8_kv_cache_hkv_amd.build``
or ``__graft_entry__.build()``); importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhkv.so")

HKV_OK = 0
STATUS_NAMES = {0: "HKV_OK", -1: "HKV_ERR_INVALID_VALUE", -2: "HKV_ERR_UNSUPPORTED", -3: "HKV_ERR_NULL_POINTER",
                -4: "HKV_ERR_CAPACITY", -5: "HKV_ERR_WORKSPACE", -6: "HKV_ERR_HIP", -7: "HKV_ERR_ALIGNMENT",
                -8: "HKV_ERR_OUT_OF_MEMORY"}
KERNELS = {"append": 0, "append_ring": 1, "decode": 2, "decode_sparse": 3, "topk_score": 4, "topk_select": 5,
           "append_decode": 6, "sparse_compact": 7, "decode_compact": 8}
EXPORTS = ["hkv_create", "hkv_destroy", "hkv_cache_sizes", "hkv_sizes", "hkv_header_table_bytes", "hkv_workspace_bytes",
           "hkv_append", "hkv_decode_attn", "hkv_decode_attn_noalloc", "hkv_append_decode",
           "hkv_sparse_store_bytes", "hkv_sparse_compact", "hkv_decode_attn_compact", "hkv_topk_select", "hkv_status_string",
           "hkv_timing_enable",
           "hkv_timing_read", "hkv_last_error_detail", "hkv_read_probe", "hkv_plan_override", "hkv_phase_stamps"]


class HKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.hkv_last_error_detail().decode() if status == -6 else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({_status_text(status)}) {detail}".rstrip())


class BlockHeader(ctypes.Structure):
    _fields_ = [("phys_block", ctypes.c_int32), ("n_valid", ctypes.c_int32),
                ("logical_block", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_phys_blocks", ctypes.c_int32), ("hot", ctypes.c_void_p), ("tail", ctypes.c_void_p),
                ("cold", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("headers", ctypes.c_void_p),
                ("seq_len_dev", ctypes.c_void_p), ("seq_len_host", ctypes.c_void_p),
                ("quant_err", ctypes.c_void_p), ("entropy", ctypes.c_void_p)]


class CacheSizes(ctypes.Structure):
    _fields_ = [("hot", ctypes.c_size_t), ("tail", ctypes.c_size_t), ("cold", ctypes.c_size_t),
                ("scales", ctypes.c_size_t), ("headers", ctypes.c_size_t), ("seq_len", ctypes.c_size_t),
                ("max_blocks_per_seq", ctypes.c_int32), ("num_phys_blocks", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libhkv.so is not built ({LIB_PATH}); run __graft_entry__.build() first")
    # torch carries its own HIP runtime (soname libamdhip64.so.7).  Load it first so that libhkv's
    # libamdhip64.so.7 dependency binds to that same runtime: two HIP runtimes in one process
    # fight over the device (hipErrorNoDevice) and could not share torch's memory and streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "hkv_create": [i32, i32, i32, i32, i32, ctypes.POINTER(vp)],
        "hkv_destroy": [vp],
        "hkv_cache_sizes": [vp, i32, i64, i64, ctypes.POINTER(CacheSizes)],
        "hkv_sizes": [vp, i32, i32, i32, ctypes.POINTER(sz)],
        "hkv_header_table_bytes": [i32, i32, i64, ctypes.POINTER(i64), ctypes.POINTER(sz)],
        "hkv_workspace_bytes": [vp, ctypes.POINTER(CacheDesc), i32, i32, ctypes.POINTER(sz)],
        "hkv_append": [vp, ctypes.POINTER(CacheDesc), vp, vp, vp, i32, vp],
        "hkv_decode_attn": [vp, ctypes.POINTER(CacheDesc), vp, i32, vp, i32, vp, vp, vp, sz, vp],
        "hkv_decode_attn_noalloc": [vp, ctypes.POINTER(CacheDesc), vp, i32, vp, i32, vp, vp, vp],
        "hkv_append_decode": [vp, ctypes.POINTER(CacheDesc), vp, vp, vp, i32, vp, vp, vp, sz, vp],
        "hkv_topk_select": [vp, ctypes.POINTER(CacheDesc), vp, i32, i32, vp, vp, sz, vp],
        "hkv_sparse_store_bytes": [vp, i32, i32, ctypes.POINTER(sz)],
        "hkv_sparse_compact": [vp, ctypes.POINTER(CacheDesc), vp, i32, vp, sz, vp],
        "hkv_decode_attn_compact": [vp, ctypes.POINTER(CacheDesc), vp, i32, vp, i32, vp, vp, vp, sz, vp],
        "hkv_timing_enable": [vp, i32],
        "hkv_timing_read": [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64), i32],
        "hkv_read_probe": [vp, sz, i32, i32, vp, vp],
        "hkv_plan_override": [vp, i32, i32],
        "hkv_phase_stamps": [vp, vp, sz],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.hkv_status_string.argtypes = [ctypes.c_int]
    lib.hkv_status_string.restype = ctypes.c_char_p
    lib.hkv_last_error_detail.argtypes = []
    lib.hkv_last_error_detail.restype = ctypes.c_char_p
    return lib


_lib = _load()


def _status_text(status: int) -> str:
    return _lib.hkv_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != HKV_OK:
        raise HKVError(status, where)


def _ptr(t) -> Optional[int]:
    """Raw device (or host) address of a torch tensor / numpy array / None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


# ----------------------------------------------------------------------------- C-ABI calls
def hkv_status_string(status: int) -> str:
    return _status_text(status)


def hkv_last_error_detail() -> str:
    return _lib.hkv_last_error_detail().decode()


def hkv_create(n_kv_heads: int, head_dim: int, hot_tokens: int = 32, block_size: int = 64,
               quant_bits: int = 8) -> int:
    h = ctypes.c_void_p()
    _check(_lib.hkv_create(n_kv_heads, head_dim, hot_tokens, block_size, quant_bits, ctypes.byref(h)), "hkv_create")
    return h.value


def hkv_destroy(handle: int) -> None:
    _check(_lib.hkv_destroy(handle), "hkv_destroy")


def hkv_cache_sizes(handle: int, batch: int, max_tokens_per_seq: int, num_phys_blocks: int = 0) -> CacheSizes:
    out = CacheSizes()
    _check(_lib.hkv_cache_sizes(handle, batch, max_tokens_per_seq, num_phys_blocks, ctypes.byref(out)),
           "hkv_cache_sizes")
    return out


def hkv_sizes(handle: int, batch: int, max_tokens_per_seq: int, num_phys_blocks: int = 0):
    """Byte counts (hot, tail, cold, scales, headers, seq_len) as a tuple."""
    out = (ctypes.c_size_t * 6)()
    _check(_lib.hkv_sizes(handle, batch, max_tokens_per_seq, num_phys_blocks, out), "hkv_sizes")
    return tuple(int(x) for x in out)


def hkv_header_table_bytes(hot_tokens: int, block_size: int, total_tokens: int):
    nb, by = ctypes.c_int64(), ctypes.c_size_t()
    _check(_lib.hkv_header_table_bytes(hot_tokens, block_size, total_tokens, ctypes.byref(nb), ctypes.byref(by)),
           "hkv_header_table_bytes")
    return nb.value, by.value


def hkv_workspace_bytes(handle: int, desc: CacheDesc, n_q_heads: int, k_sel: int = 0) -> int:
    out = ctypes.c_size_t()
    _check(_lib.hkv_workspace_bytes(handle, ctypes.byref(desc), n_q_heads, k_sel, ctypes.byref(out)),
           "hkv_workspace_bytes")
    return out.value


def hkv_append(handle: int, desc: CacheDesc, k_new, v_new, n_new_host: np.ndarray, stream=None) -> None:
    n_new = np.ascontiguousarray(n_new_host, dtype=np.int32)
    max_n_new = int(k_new.shape[1]) if k_new is not None else 0
    _check(_lib.hkv_append(handle, ctypes.byref(desc), _ptr(k_new), _ptr(v_new), n_new.ctypes.data, max_n_new,
                           _stream(stream)), "hkv_append")


def hkv_decode_attn(handle: int, desc: CacheDesc, q, out, workspace, lse=None, sel_idx=None, k_sel: int = 0,
                    stream=None) -> None:
    _check(_lib.hkv_decode_attn(handle, ctypes.byref(desc), _ptr(q), int(q.shape[1]), _ptr(sel_idx),
                                int(k_sel), _ptr(out), _ptr(lse), _ptr(workspace),
                                int(workspace.numel() * workspace.element_size()), _stream(stream)),
           "hkv_decode_attn")


def hkv_decode_attn_noalloc(handle: int, desc: CacheDesc, q, out, lse=None, sel_idx=None, k_sel: int = 0,
                            stream=None) -> None:
    _check(_lib.hkv_decode_attn_noalloc(handle, ctypes.byref(desc), _ptr(q), int(q.shape[1]), _ptr(sel_idx),
                                        int(k_sel), _ptr(out), _ptr(lse), _stream(stream)),
           "hkv_decode_attn_noalloc")


def hkv_append_decode(handle: int, desc: CacheDesc, k_new, v_new, q, out, workspace, lse=None, stream=None) -> None:
    _check(_lib.hkv_append_decode(handle, ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(q), int(q.shape[1]),
                                  _ptr(out), _ptr(lse), _ptr(workspace),
                                  int(workspace.numel() * workspace.element_size()), _stream(stream)),
           "hkv_append_decode")


def hkv_topk_select(handle: int, desc: CacheDesc, q, k: int, out_idx, workspace, stream=None) -> None:
    _check(_lib.hkv_topk_select(handle, ctypes.byref(desc), _ptr(q), int(q.shape[1]), int(k), _ptr(out_idx),
                                _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                _stream(stream)), "hkv_topk_select")


def hkv_read_probe(src, nbytes: int, workgroups: int, threads: int, sink, stream=None) -> None:
    """One launch reading nbytes of src (a device tensor) once (measurement aid)."""
    _check(_lib.hkv_read_probe(_ptr(src), int(nbytes), int(workgroups), int(threads), _ptr(sink), _stream(stream)),
           "hkv_read_probe")


def hkv_sparse_store_bytes(handle: int, batch: int, k_sel: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.hkv_sparse_store_bytes(handle, batch, k_sel, ctypes.byref(out)), "hkv_sparse_store_bytes")
    return out.value


def hkv_sparse_compact(handle: int, desc: CacheDesc, sel_idx, k_sel: int, store, stream=None) -> None:
    _check(_lib.hkv_sparse_compact(handle, ctypes.byref(desc), _ptr(sel_idx), int(k_sel), _ptr(store),
                                   int(store.numel() * store.element_size()), _stream(stream)), "hkv_sparse_compact")


def hkv_decode_attn_compact(handle: int, desc: CacheDesc, store, k_sel: int, q, out, workspace, lse=None,
                            stream=None) -> None:
    _check(_lib.hkv_decode_attn_compact(handle, ctypes.byref(desc), _ptr(store), int(k_sel), _ptr(q), int(q.shape[1]),
                                        _ptr(out), _ptr(lse), _ptr(workspace),
                                        int(workspace.numel() * workspace.element_size()), _stream(stream)),
           "hkv_decode_attn_compact")


def hkv_phase_stamps(handle: int, buf=None) -> None:
    """Per-workgroup phase timestamps of the handle's decode launches into `buf` (uint64 / int64
    device tensor, 8 per workgroup), or off with None."""
    if buf is None:
        _check(_lib.hkv_phase_stamps(handle, None, 0), "hkv_phase_stamps")
    else:
        _check(_lib.hkv_phase_stamps(handle, _ptr(buf), int(buf.numel() * buf.element_size())), "hkv_phase_stamps")


def hkv_plan_override(handle: int, nsplit: int = 0, claim_workgroups: int = 0) -> None:
    _check(_lib.hkv_plan_override(handle, int(nsplit), int(claim_workgroups)), "hkv_plan_override")


def hkv_timing_enable(handle: int, enable: bool = True) -> None:
    _check(_lib.hkv_timing_enable(handle, 1 if enable else 0), "hkv_timing_enable")


def hkv_timing_read(handle: int, kernel: str, reset: bool = False):
    ms, cnt = ctypes.c_double(), ctypes.c_int64()
    _check(_lib.hkv_timing_read(handle, KERNELS[kernel], ctypes.byref(ms), ctypes.byref(cnt), 1 if reset else 0),
           "hkv_timing_read")
    return ms.value, cnt.value


# ----------------------------------------------------------------------------- buffer owner
class HybridKVCache:
    """Owns one layer's cache buffers (torch, on ``device``) and its descriptor.

    ``phys_ids`` (optional, int array [batch, max_blocks_per_seq]) places each
    logical block at a physical block id; by default blocks are laid out
    densely in (sequence, logical block) order.
    """

    def __init__(self, n_kv_heads: int, head_dim: int, batch: int, max_tokens_per_seq: int, *,
                 hot_tokens: int = 32, block_size: int = 64, quant_bits: int = 8, num_phys_blocks: int = 0,
                 phys_ids: Optional[np.ndarray] = None, device: str = "cuda"):
        import torch
        self.torch = torch
        self.H, self.D, self.T, self.S = n_kv_heads, head_dim, hot_tokens, block_size
        self.quant_bits = quant_bits
        self.batch = batch
        self.handle = hkv_create(n_kv_heads, head_dim, hot_tokens, block_size, quant_bits)
        sz = hkv_cache_sizes(self.handle, batch, max_tokens_per_seq, num_phys_blocks)
        self.max_blocks = sz.max_blocks_per_seq
        self.num_phys = sz.num_phys_blocks
        dev = torch.device(device)
        self.hot = torch.zeros(sz.hot // 2, dtype=torch.float16, device=dev)
        self.tail = torch.zeros(sz.tail // 2, dtype=torch.float16, device=dev)
        self.cold = torch.zeros(max(sz.cold, 16), dtype=torch.int8, device=dev)
        self.scales = torch.zeros(max(sz.scales // 4, 4), dtype=torch.float32, device=dev)
        hdr = np.zeros((batch, max(self.max_blocks, 1), 4), dtype=np.int32)
        if phys_ids is None:
            phys_ids = np.arange(batch * self.max_blocks, dtype=np.int64).reshape(batch, self.max_blocks)
        hdr[:, :self.max_blocks, 0] = np.asarray(phys_ids, dtype=np.int64).reshape(batch, self.max_blocks)
        self.headers = torch.from_numpy(hdr.reshape(-1)).to(dev)
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.seq_len_host = np.zeros(batch, dtype=np.int32)
        self.desc = CacheDesc(batch, self.max_blocks, self.num_phys, self.hot.data_ptr(), self.tail.data_ptr(),
                              self.cold.data_ptr(), self.scales.data_ptr(), self.headers.data_ptr(),
                              self.seq_len.data_ptr(), self.seq_len_host.ctypes.data)
        self._ws = None

    # -- debug statistics (optional descriptor fields)
    def enable_debug(self, n_q_heads: int):
        """Allocate and register the debug statistics: quant_err fp32 [P, H, 2] (written by appends for
        every tile they code) and entropy fp32 [batch, n_q_heads] (written by every decode).  Returns
        (quant_err, entropy)."""
        torch = self.torch
        self.quant_err = torch.zeros(max(self.num_phys * self.H * 2, 1), dtype=torch.float32, device=self.hot.device)
        self.entropy = torch.full((self.batch, n_q_heads), float("nan"), dtype=torch.float32, device=self.hot.device)
        self.desc.quant_err = self.quant_err.data_ptr()
        self.desc.entropy = self.entropy.data_ptr()
        return self.quant_err, self.entropy

    def disable_debug(self) -> None:
        self.desc.quant_err = None
        self.desc.entropy = None

    # -- C-ABI wrappers bound to this cache
    def workspace(self, n_q_heads: int, k_sel: int = 0):
        need = hkv_workspace_bytes(self.handle, self.desc, n_q_heads, k_sel)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self.torch.zeros(need, dtype=self.torch.uint8, device=self.hot.device)
        return self._ws

    def append(self, k_new, v_new, n_new: Optional[Sequence[int]] = None, stream=None) -> None:
        if n_new is None:
            n_new = np.full(self.batch, int(k_new.shape[1]), dtype=np.int32)
        hkv_append(self.handle, self.desc, k_new, v_new, np.asarray(n_new, dtype=np.int32), stream)

    def decode(self, q, out=None, lse=None, sel_idx=None, k_sel: int = 0, workspace=None, stream=None):
        torch = self.torch
        if out is None:
            out = torch.empty_like(q)
        ws = workspace if workspace is not None else self.workspace(int(q.shape[1]), k_sel)
        hkv_decode_attn(self.handle, self.desc, q, out, ws, lse=lse, sel_idx=sel_idx, k_sel=k_sel, stream=stream)
        return out

    def append_decode(self, k_new, v_new, q, out=None, lse=None, workspace=None, stream=None):
        """One decode step: append one token per sequence (k_new/v_new [batch, H, D] or [batch, 1, H, D])
        and decode q against the updated cache, in one launch."""
        torch = self.torch
        if out is None:
            out = torch.empty_like(q)
        ws = workspace if workspace is not None else self.workspace(int(q.shape[1]))
        hkv_append_decode(self.handle, self.desc, k_new, v_new, q, out, ws, lse=lse, stream=stream)
        return out

    def sparse_store(self, sel_idx, k_sel: int, store=None, stream=None):
        """Build a compacted sparse store of the selection sel_idx [batch, H, k_sel]; returns the store."""
        torch = self.torch
        if store is None:
            store = torch.zeros(hkv_sparse_store_bytes(self.handle, self.batch, k_sel), dtype=torch.uint8,
                                device=self.hot.device)
        hkv_sparse_compact(self.handle, self.desc, sel_idx, k_sel, store, stream=stream)
        return store

    def decode_store(self, q, store, k_sel: int, out=None, lse=None, workspace=None, stream=None):
        """Decode over the hot zone plus a compacted sparse store."""
        torch = self.torch
        if out is None:
            out = torch.empty_like(q)
        ws = workspace if workspace is not None else self.workspace(int(q.shape[1]), k_sel)
        hkv_decode_attn_compact(self.handle, self.desc, store, k_sel, q, out, ws, lse=lse, stream=stream)
        return out

    def store_rows(self, store, k_sel: int):
        """Host view of a store: (counts [B, H], k rows [B, H, U*64, D], v rows, scales [B, H, U*64, 2])."""
        B, H, S, D = self.batch, self.H, self.S, self.D
        U = -(-k_sel // S)
        raw = store.cpu().numpy().view(np.uint8)
        bh = B * H
        scales_off = -(-(bh * 4) // 256) * 256
        units_off = -(-(scales_off + bh * U * S * 8) // 256) * 256
        counts = raw[:bh * 4].view(np.int32).reshape(B, H)
        scales = raw[scales_off:scales_off + bh * U * S * 8].view(np.float32).reshape(B, H, U * S, 2)
        TB = self._tile_bytes()
        tiles = raw[units_off:units_off + bh * U * 2 * TB].reshape(bh * U, 2, TB)
        rows = self._tiles_to_rows(tiles).reshape(B, H, U, 2, S, D)
        k_rows = rows[:, :, :, 0].reshape(B, H, U * S, D)
        v_rows = rows[:, :, :, 1].reshape(B, H, U * S, D)
        return counts, k_rows, v_rows, scales

    def topk(self, q, k: int, out_idx=None, workspace=None, stream=None):
        torch = self.torch
        if out_idx is None:
            out_idx = torch.empty((self.batch, self.H, k), dtype=torch.int32, device=q.device)
        ws = workspace if workspace is not None else self.workspace(int(q.shape[1]), k)
        hkv_topk_select(self.handle, self.desc, q, k, out_idx, ws, stream=stream)
        return out_idx

    # -- layout helpers for inspection (host numpy views of device buffers)
    def _tile_elems(self) -> int:
        """Elements per 16-byte tile chunk: 16 (8-bit codes), 32 (4-bit codes), 8 (fp16 values)."""
        return {8: 16, 4: 32, 0: 8}[self.quant_bits]

    def _tile_bytes(self) -> int:
        n = self.S * self.D
        return n * 2 if self.quant_bits == 0 else n * self.quant_bits // 8

    def _unpack(self, raw: np.ndarray) -> np.ndarray:
        """Tile bytes [..., TB] -> elements in chunk order [..., S*D]: codes (int8), or fp16 values."""
        if self.quant_bits == 8:
            return (raw.view(np.uint8) ^ 0x80).view(np.int8)  # offset binary: byte = code + 128
        if self.quant_bits == 0:
            return raw.view(np.float16)
        u = raw.view(np.uint8)
        w = u.reshape(u.shape[:-1] + (u.shape[-1] // 4, 4))  # 32-bit words of four bytes
        out = np.empty(w.shape[:-1] + (8,), dtype=np.int8)
        out[..., :4] = (w & 0x0F).astype(np.int8) - 8  # offset binary, planar: elements 8j..8j+3 low nibbles
        out[..., 4:] = (w >> 4).astype(np.int8) - 8    # elements 8j+4..8j+7: the high nibbles
        return out.reshape(u.shape[:-1] + (u.shape[-1] * 2,))

    def _tiles_to_rows(self, tiles: np.ndarray) -> np.ndarray:
        """[N, 2, TB] tile bytes of (block, kv-head) pairs -> [N, 2, S, D] codes (token, channel order)."""
        S, D, E = self.S, self.D, self._tile_elems()
        el = self._unpack(np.ascontiguousarray(tiles))
        N = tiles.shape[0]
        out = np.empty((N, 2, S, D), dtype=el.dtype)
        out[:, 0] = el[:, 0].reshape(N, D // E, S, E).transpose(0, 2, 1, 3).reshape(N, S, D)   # chunk (kc, t)
        out[:, 1] = el[:, 1].reshape(N, S // E, D, E).transpose(0, 1, 3, 2).reshape(N, S, D)   # chunk (vc, c)
        return out

    def cold_codes(self) -> np.ndarray:
        """[P, H, 2, S, D] cold contents in (token, channel) order, un-doing the streaming tile layouts:
        int8 codes (8 and 4 bits) or fp16 values (quant_bits 0)."""
        TB = self._tile_bytes()
        raw = self.cold.cpu().numpy().view(np.uint8)[: self.num_phys * self.H * 2 * TB]
        tiles = raw.reshape(self.num_phys * self.H, 2, TB)
        return self._tiles_to_rows(tiles).reshape(self.num_phys, self.H, 2, self.S, self.D)

    def cold_codes_of(self, phys: Sequence[int]) -> np.ndarray:
        """[len(phys), H, 2, S, D] cold contents of selected physical blocks only."""
        TB = self._tile_bytes()
        blk = self.H * 2 * TB
        raws = [self.cold[int(p) * blk:(int(p) + 1) * blk].cpu().numpy().view(np.uint8) for p in phys]
        tiles = np.stack(raws).reshape(len(phys) * self.H, 2, TB)
        return self._tiles_to_rows(tiles).reshape(len(phys), self.H, 2, self.S, self.D)

    def scale_array(self) -> np.ndarray:
        return self.scales.cpu().numpy()[: self.num_phys * self.H * 2].reshape(self.num_phys, self.H, 2)

    def header_array(self) -> np.ndarray:
        return self.headers.cpu().numpy().reshape(self.batch, -1, 4)[:, :self.max_blocks]

    def hot_array(self) -> np.ndarray:
        return self.hot.cpu().numpy().reshape(self.batch, self.H, self.T, 2, self.D)

    def close(self) -> None:
        if self.handle:
            hkv_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
