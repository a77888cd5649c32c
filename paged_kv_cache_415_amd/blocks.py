"""Python binding of the native block manager with a prefix cache
(include/pa_blocks.h): argument marshalling only."""

from __future__ import annotations

import ctypes

import numpy as np

from . import PagedAttentionError, library

_i32, _i64, _u64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p
_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)
OUT_OF_BLOCKS = 5


def _setup(lib):
    lib.pa_bm_create.argtypes = [_i32, _i32, _P32, ctypes.POINTER(_vp)]
    lib.pa_bm_create.restype = _i32
    lib.pa_bm_destroy.argtypes = [_vp]
    lib.pa_bm_destroy.restype = None
    for name in ("pa_bm_num_free", "pa_bm_num_evictable", "pa_bm_num_cached"):
        getattr(lib, name).argtypes = [_vp]
        getattr(lib, name).restype = _i32
    lib.pa_bm_ref_count.argtypes = [_vp, _i32]
    lib.pa_bm_ref_count.restype = _i32
    lib.pa_bm_allocate_prompt.argtypes = [_vp, _u64, _P32, _i32, _P32, _i32, _P32, _P32]
    lib.pa_bm_append.argtypes = [_vp, _P32, _i32, _i32, _i32, _P32]
    lib.pa_bm_register_blocks.argtypes = [_vp, _u64, _P32, _i32, _P32, _i32, _P32]
    lib.pa_bm_fork.argtypes = [_vp, _P32, _i32]
    lib.pa_bm_copy_on_write.argtypes = [_vp, _P32, _i32, _i32, _P64]
    lib.pa_bm_release.argtypes = [_vp, _P32, _i32]
    for name in ("pa_bm_allocate_prompt", "pa_bm_append", "pa_bm_fork", "pa_bm_copy_on_write",
                 "pa_bm_release", "pa_bm_register_blocks"):
        getattr(lib, name).restype = _i32
    return lib


_lib = _setup(library())


class OutOfBlocks(PagedAttentionError):
    pass


def _check(status: int) -> None:
    if status == OUT_OF_BLOCKS:
        raise OutOfBlocks(status, _lib.pa_last_error().decode())
    if status != 0:
        raise PagedAttentionError(status, _lib.pa_last_error().decode())


def _arr(values) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_P32)


class BlockManager:
    """Owner of one native block manager handle; tables are Python lists of ints."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.block_size = block_size
        handle = _vp()
        order_arr = None if order is None else _arr(order)
        if order_arr is not None and order_arr.size != num_blocks:
            raise ValueError("order must hold num_blocks entries")
        _check(_lib.pa_bm_create(num_blocks, block_size,
                                 None if order_arr is None else _p32(order_arr),
                                 ctypes.byref(handle)))
        self._h = handle
        self._destroy = _lib.pa_bm_destroy      # kept for interpreter shutdown

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def num_free(self) -> int:
        return _lib.pa_bm_num_free(self._h)

    def num_evictable(self) -> int:
        return _lib.pa_bm_num_evictable(self._h)

    def num_cached(self) -> int:
        return _lib.pa_bm_num_cached(self._h)

    def ref_count(self, block: int) -> int:
        return _lib.pa_bm_ref_count(self._h, block)

    def allocate_prompt(self, namespace: int, tokens):
        """Blocks for a prompt and the number of leading prefix-cache hits."""
        tok = _arr(tokens)
        cap = -(-tok.size // self.block_size)
        out = np.zeros(max(cap, 1), np.int32)
        n, hits = _i32(), _i32()
        _check(_lib.pa_bm_allocate_prompt(self._h, int(namespace) & (2**64 - 1), _p32(tok), tok.size,
                                          _p32(out), cap, ctypes.byref(n), ctypes.byref(hits)))
        return out[:n.value].tolist(), hits.value

    def register_blocks(self, namespace: int, tokens, table: list) -> int:
        """Cache the full blocks of a sequence's tokens that its table holds."""
        tok = _arr(tokens)
        buf = _arr(table) if table else np.zeros(1, np.int32)
        n = _i32()
        _check(_lib.pa_bm_register_blocks(self._h, int(namespace) & (2**64 - 1), _p32(tok), tok.size,
                                          _p32(buf), len(table), ctypes.byref(n)))
        return n.value

    def append(self, table: list, new_len: int) -> None:
        need = -(-new_len // self.block_size)
        buf = np.zeros(max(need, len(table), 1), np.int32)
        buf[:len(table)] = table
        n = _i32()
        _check(_lib.pa_bm_append(self._h, _p32(buf), len(table), buf.size, new_len, ctypes.byref(n)))
        table[:] = buf[:n.value].tolist()

    def fork(self, table: list) -> list:
        buf = _arr(table) if table else np.zeros(1, np.int32)
        _check(_lib.pa_bm_fork(self._h, _p32(buf), len(table)))
        return list(table)

    def copy_on_write(self, table: list, logical: int):
        buf = _arr(table)
        pair = (ctypes.c_int64 * 2)()
        _check(_lib.pa_bm_copy_on_write(self._h, _p32(buf), len(table), logical, pair))
        if pair[0] < 0:
            return None
        table[logical] = int(buf[logical])
        return (int(pair[0]), int(pair[1]))

    def release(self, table: list) -> None:
        buf = _arr(table) if table else np.zeros(1, np.int32)
        _check(_lib.pa_bm_release(self._h, _p32(buf), len(table)))


__all__ = ["BlockManager", "OutOfBlocks"]
