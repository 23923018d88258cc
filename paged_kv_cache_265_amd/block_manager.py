"""Binding of the native block manager (include/pkv_block_manager.h).

Argument marshalling only: every operation runs in libpkv.so's C++ manager.
"""

from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .pkv import PkvError, load_library

NO_BLOCKS = -5

SYMBOLS = (
    "pkv_bm_create", "pkv_bm_destroy", "pkv_bm_num_free", "pkv_bm_add_sequence", "pkv_bm_fork",
    "pkv_bm_append", "pkv_bm_commit_prompt", "pkv_bm_free_sequence", "pkv_bm_context_len",
    "pkv_bm_block_table", "pkv_bm_refcount", "pkv_bm_free_queue",
)

_ready = False


def _lib():
    global _ready
    lib = load_library()
    if not _ready:
        P, I, LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
        lib.pkv_bm_create.argtypes = [I, I]
        lib.pkv_bm_create.restype = P
        lib.pkv_bm_destroy.argtypes = [P]
        lib.pkv_bm_destroy.restype = None
        lib.pkv_bm_num_free.argtypes = [P]
        lib.pkv_bm_add_sequence.argtypes = [P, I, P, I, P]
        lib.pkv_bm_fork.argtypes = [P, I, I]
        lib.pkv_bm_append.argtypes = [P, I, I, P, P, I, P]
        lib.pkv_bm_commit_prompt.argtypes = [P, I, P, I, P]
        lib.pkv_bm_free_sequence.argtypes = [P, I]
        lib.pkv_bm_context_len.argtypes = [P, I]
        lib.pkv_bm_context_len.restype = LL
        lib.pkv_bm_block_table.argtypes = [P, I, P, I, ctypes.c_int32, P]
        lib.pkv_bm_refcount.argtypes = [P, I]
        lib.pkv_bm_free_queue.argtypes = [P, P, I]
        for f in ("pkv_bm_num_free", "pkv_bm_add_sequence", "pkv_bm_fork", "pkv_bm_append",
                  "pkv_bm_commit_prompt", "pkv_bm_free_sequence", "pkv_bm_block_table", "pkv_bm_refcount",
                  "pkv_bm_free_queue"):
            getattr(lib, f).restype = I
        _ready = True
    return lib


def _check(rc: int) -> int:
    if rc < 0:
        lib = load_library()
        if rc == NO_BLOCKS:
            raise MemoryError(lib.pkv_last_error().decode())
        raise PkvError(rc, f"{lib.pkv_error_string(rc).decode()}: {lib.pkv_last_error().decode()}")
    return rc


def _i32(tokens: Optional[Sequence[int]]):
    if tokens is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    return a, len(a)


class BlockManager:
    """Free-block queue, block tables, reference counts, copy-on-write and prefix
    caching of a paged KV pool (host side)."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = _lib()
        self._h = self._lib.pkv_bm_create(num_blocks, block_size)
        if not self._h:
            raise PkvError(-1, load_library().pkv_last_error().decode())
        self.num_blocks = num_blocks
        self.block_size = block_size

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def num_free(self) -> int:
        return _check(self._lib.pkv_bm_num_free(self._h))

    def add_sequence(self, seq: int, prompt: Optional[Sequence[int]] = None) -> int:
        a, n = _i32(prompt)
        cached = ctypes.c_int(0)
        _check(self._lib.pkv_bm_add_sequence(self._h, seq, None if a is None else a.ctypes.data, n,
                                             ctypes.byref(cached)))
        return cached.value

    def fork(self, parent: int, child: int) -> None:
        _check(self._lib.pkv_bm_fork(self._h, parent, child))

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots = np.zeros(max(n, 1), dtype=np.int64)
        copies = np.zeros(2, dtype=np.int64)
        nc = ctypes.c_int(0)
        _check(self._lib.pkv_bm_append(self._h, seq, n, slots.ctypes.data, copies.ctypes.data, 1, ctypes.byref(nc)))
        return slots[:n].tolist(), [(int(copies[0]), int(copies[1]))] if nc.value else []

    def commit_prompt(self, seq: int, prompt: Sequence[int]) -> int:
        a, n = _i32(prompt)
        added = ctypes.c_int(0)
        _check(self._lib.pkv_bm_commit_prompt(self._h, seq, a.ctypes.data if n else None, n, ctypes.byref(added)))
        return added.value

    def free_sequence(self, seq: int) -> None:
        _check(self._lib.pkv_bm_free_sequence(self._h, seq))

    def context_len(self, seq: int) -> int:
        return _check(int(self._lib.pkv_bm_context_len(self._h, seq)))

    def block_table(self, seq: int, max_blocks: Optional[int] = None, pad: int = 0x7FFFFFFF) -> List[int]:
        if max_blocks is None:
            max_blocks = -(-self.context_len(seq) // self.block_size)
        out = np.zeros(max(max_blocks, 1), dtype=np.int32)
        nb = ctypes.c_int(0)
        _check(self._lib.pkv_bm_block_table(self._h, seq, out.ctypes.data, max_blocks, pad, ctypes.byref(nb)))
        return out[:nb.value].tolist()

    def refcount(self, block: int) -> int:
        return _check(self._lib.pkv_bm_refcount(self._h, block))

    def free_order(self) -> List[int]:
        out = np.zeros(self.num_blocks, dtype=np.int32)
        k = _check(self._lib.pkv_bm_free_queue(self._h, out.ctypes.data, self.num_blocks))
        return out[:k].tolist()
