"""Python handle on the native host block allocator (kvs_alloc_* in libkvs)."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

from ._lib import lib, check, KvsError, KVS_E_NOBLOCKS


class BlockAllocator:
    """FIFO free list + reference counts + copy-on-write, implemented in C++."""

    def __init__(self, num_blocks: int, initial_free_order: Optional[Sequence[int]] = None):
        h = ctypes.c_void_p()
        if initial_free_order is None:
            check(lib.kvs_alloc_create(int(num_blocks), None, 0, ctypes.byref(h)))
        else:
            arr = (ctypes.c_int32 * len(initial_free_order))(*[int(b) for b in initial_free_order])
            check(lib.kvs_alloc_create(int(num_blocks), arr, len(initial_free_order), ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            lib.kvs_alloc_destroy(h)
            self._h = None

    def alloc(self) -> int:
        b = ctypes.c_int32()
        check(lib.kvs_alloc_block(self._h, ctypes.byref(b)))
        return b.value

    def alloc_n(self, n: int) -> list:
        return [self.alloc() for _ in range(n)]

    def incref(self, b: int) -> None:
        check(lib.kvs_alloc_incref(self._h, int(b)))

    def decref(self, b: int) -> None:
        check(lib.kvs_alloc_decref(self._h, int(b)))

    def refcount(self, b: int) -> int:
        return check(lib.kvs_alloc_refcount(self._h, int(b)))

    def num_free(self) -> int:
        return check(lib.kvs_alloc_num_free(self._h))

    def free_list(self) -> list:
        n = self.num_free()
        arr = (ctypes.c_int32 * max(n, 1))()
        m = check(lib.kvs_alloc_free_list(self._h, arr, n))
        return list(arr[:m])

    def cow(self, b: int):
        """(block to write, copied?) - a shared block is swapped for a fresh one."""
        out = ctypes.c_int32()
        copied = ctypes.c_int()
        check(lib.kvs_alloc_cow(self._h, int(b), ctypes.byref(out), ctypes.byref(copied)))
        return out.value, bool(copied.value)


__all__ = ["BlockAllocator", "KvsError", "KVS_E_NOBLOCKS"]
