"""ctypes binding of the library's host-side block manager (include/pa_block_manager.h).

Argument marshalling only: every operation runs in the C++ library.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import binding

HASH_SHA256 = 0
HASH_FNV1A64 = 1
ERR_NO_BLOCKS = -5
ERR_REQUEST = -6

EXPORTED = ("pa_bm_create", "pa_bm_destroy", "pa_bm_add_request", "pa_bm_fork",
            "pa_bm_append_token", "pa_bm_free_request", "pa_bm_decode_step",
            "pa_bm_block_table", "pa_bm_num_tokens", "pa_bm_num_free_blocks",
            "pa_bm_num_cached_blocks", "pa_bm_refcount", "pa_bm_free_queue", "pa_bm_lookup",
            "pa_bm_block_key", "pa_bm_sha256")

_declared = False


class PoolExhausted(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _declared
    L = binding.lib()
    if _declared:
        return L
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P32 = ctypes.POINTER(ctypes.c_int32)
    P64 = ctypes.POINTER(ctypes.c_int64)
    L.pa_bm_create.argtypes = [i64, i32, i32, vp]
    L.pa_bm_create.restype = vp
    L.pa_bm_destroy.argtypes = [vp]
    L.pa_bm_destroy.restype = None
    L.pa_bm_add_request.argtypes = [vp, i64, vp, i32, vp, i32, P32]
    L.pa_bm_add_request.restype = ctypes.c_int
    L.pa_bm_fork.argtypes = [vp, i64, i64]
    L.pa_bm_fork.restype = ctypes.c_int
    L.pa_bm_append_token.argtypes = [vp, i64, i32, P64, P64, P64]
    L.pa_bm_append_token.restype = ctypes.c_int
    L.pa_bm_free_request.argtypes = [vp, i64]
    L.pa_bm_free_request.restype = ctypes.c_int
    L.pa_bm_decode_step.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, vp, P32]
    L.pa_bm_decode_step.restype = ctypes.c_int
    L.pa_bm_block_table.argtypes = [vp, i64, vp, i32]
    L.pa_bm_block_table.restype = i32
    L.pa_bm_num_tokens.argtypes = [vp, i64]
    L.pa_bm_num_tokens.restype = i32
    L.pa_bm_num_free_blocks.argtypes = [vp]
    L.pa_bm_num_free_blocks.restype = i64
    L.pa_bm_num_cached_blocks.argtypes = [vp]
    L.pa_bm_num_cached_blocks.restype = i64
    L.pa_bm_refcount.argtypes = [vp, i64]
    L.pa_bm_refcount.restype = i32
    L.pa_bm_free_queue.argtypes = [vp, vp, i64]
    L.pa_bm_free_queue.restype = i64
    L.pa_bm_lookup.argtypes = [vp, vp]
    L.pa_bm_lookup.restype = i64
    L.pa_bm_block_key.argtypes = [vp, vp, i32, vp, i32, i32, vp]
    L.pa_bm_block_key.restype = ctypes.c_int
    L.pa_bm_sha256.argtypes = [vp, sz, vp]
    L.pa_bm_sha256.restype = ctypes.c_int
    _declared = True
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))


def _bytes(b: bytes) -> np.ndarray:
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


def _check(code: int, what: str) -> None:
    if code == ERR_NO_BLOCKS:
        raise PoolExhausted(f"{what}: not enough free blocks")
    if code < 0:
        raise binding.PagedKVError(code, what)


def sha256(data: bytes) -> bytes:
    buf = _bytes(data)
    out = np.zeros(32, dtype=np.uint8)
    _check(lib().pa_bm_sha256(_ptr(buf), len(data), _ptr(out)), "pa_bm_sha256")
    return out.tobytes()


def block_key(parent: bytes, tokens, extra: bytes = b"", kind: int = HASH_SHA256) -> bytes:
    p = _bytes(parent)
    t = _i32(tokens)
    e = _bytes(extra)
    out = np.zeros(32, dtype=np.uint8)
    _check(lib().pa_bm_block_key(_ptr(p), _ptr(t), t.size, _ptr(e), e.size, kind, _ptr(out)),
           "pa_bm_block_key")
    return out.tobytes()


class BlockManager:
    """A handle on one C++ block manager (see include/pa_block_manager.h)."""

    def __init__(self, num_blocks: int, block_size: int = 16, hash_kind: int = HASH_SHA256,
                 free_order=None):
        self._L = lib()
        order = None if free_order is None else _i32(free_order)
        self._order_keepalive = order
        h = self._L.pa_bm_create(int(num_blocks), int(block_size), int(hash_kind),
                                 None if order is None else _ptr(order))
        if not h:
            raise ValueError("pa_bm_create rejected its arguments")
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self) -> None:
        if self._h:
            self._L.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add_request(self, rid: int, tokens, extra: bytes = b"") -> int:
        t = _i32(tokens)
        e = _bytes(extra)
        cached = ctypes.c_int32(0)
        _check(self._L.pa_bm_add_request(self._h, int(rid), _ptr(t), t.size, _ptr(e), e.size,
                                         ctypes.byref(cached)), "pa_bm_add_request")
        return cached.value

    def fork(self, parent: int, child: int) -> None:
        _check(self._L.pa_bm_fork(self._h, int(parent), int(child)), "pa_bm_fork")

    def append_token(self, rid: int, token: int):
        slot, src, dst = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(self._L.pa_bm_append_token(self._h, int(rid), int(token), ctypes.byref(slot),
                                          ctypes.byref(src), ctypes.byref(dst)),
               "pa_bm_append_token")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def free_request(self, rid: int) -> None:
        _check(self._L.pa_bm_free_request(self._h, int(rid)), "pa_bm_free_request")

    def decode_step(self, rids, tokens, max_blocks_per_seq: int):
        """Returns (block_tables [S, MB], context_lens [S], slot_mapping [S],
        block_mapping [P, 2]) ready for the device entry points."""
        r = np.ascontiguousarray(np.asarray(rids, dtype=np.int64).reshape(-1))
        t = _i32(tokens)
        S = r.size
        tables = np.full((S, max_blocks_per_seq), -1, dtype=np.int32)
        lens = np.zeros(S, dtype=np.int32)
        slots = np.zeros(S, dtype=np.int64)
        pairs = np.zeros((max(S, 1), 2), dtype=np.int64)
        n = ctypes.c_int32(0)
        _check(self._L.pa_bm_decode_step(self._h, _ptr(r), _ptr(t), S, int(max_blocks_per_seq),
                                         _ptr(tables), _ptr(lens), _ptr(slots), _ptr(pairs),
                                         ctypes.byref(n)), "pa_bm_decode_step")
        return tables, lens, slots, pairs[:n.value].copy()

    def block_table(self, rid: int) -> list:
        n = self._L.pa_bm_block_table(self._h, int(rid), None, 0)
        _check(n, "pa_bm_block_table")
        out = np.zeros(n, dtype=np.int32)
        self._L.pa_bm_block_table(self._h, int(rid), _ptr(out), n)
        return out.tolist()

    def num_tokens(self, rid: int) -> int:
        n = self._L.pa_bm_num_tokens(self._h, int(rid))
        _check(n, "pa_bm_num_tokens")
        return n

    def num_free(self) -> int:
        return int(self._L.pa_bm_num_free_blocks(self._h))

    def num_cached(self) -> int:
        return int(self._L.pa_bm_num_cached_blocks(self._h))

    def refcount(self, block: int) -> int:
        return int(self._L.pa_bm_refcount(self._h, int(block)))

    def free_queue(self) -> list:
        n = self._L.pa_bm_free_queue(self._h, None, 0)
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._L.pa_bm_free_queue(self._h, _ptr(out), n)
        return out[:n].tolist()

    def lookup(self, key: bytes) -> int:
        k = _bytes(key)
        return int(self._L.pa_bm_lookup(self._h, _ptr(k)))
