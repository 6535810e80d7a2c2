"""Python binding of the host block manager in ``libpaged_kv.so``
(``pa_bm_*`` in ``include/paged_kv.h``): argument marshalling only; the
allocation, prefix matching, reference counting and eviction run in the
library's C++.

    bm = BlockManager(num_blocks, block_size)
    sid, cached = bm.add_sequence(token_ids)     # cached: leading tokens already in the cache
    slot = bm.append(sid, token_id)              # slot for pa_write_kv
    slots = bm.append_batch(sids, token_ids)     # one decode step's slot_mapping
    bm.block_table(sid), bm.slots(sid, start, count), bm.length(sid), bm.num_free()
    tables, lens = bm.fill_tables(sids, max_blocks_per_seq)   # host arrays for decode / prefill
    bm.free_sequence(sid)
"""
from __future__ import annotations

import ctypes

import numpy as np

from .api import PaError, load_library

__all__ = ["BlockManager", "BlockManagerError"]

PA_ERR_NO_BLOCKS, PA_ERR_NO_SEQUENCE, PA_ERR_NO_MEMORY = -8, -9, -10


class BlockManagerError(PaError):
    """Not enough free blocks, or an unknown sequence; nothing was changed."""


_SIGNED = False


def _lib():
    global _SIGNED
    lib = load_library()
    if not _SIGNED:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        p64, p32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
        sig = {
            "pa_bm_create": (vp, [i32, i32]),
            "pa_bm_destroy": (None, [vp]),
            "pa_bm_add_sequence": (ctypes.c_int, [vp, vp, i32, p64, p32]),
            "pa_bm_append": (ctypes.c_int, [vp, i64, i64, p64]),
            "pa_bm_free_sequence": (ctypes.c_int, [vp, i64]),
            "pa_bm_append_batch": (ctypes.c_int, [vp, vp, vp, i32, vp]),
            "pa_bm_length": (i32, [vp, i64]),
            "pa_bm_num_free": (i32, [vp]),
            "pa_bm_block_table": (ctypes.c_int, [vp, i64, vp, i32, p32]),
            "pa_bm_slots": (ctypes.c_int, [vp, i64, i32, i32, vp]),
            "pa_bm_fill_tables": (ctypes.c_int, [vp, vp, i32, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _SIGNED = True
    return lib


def _check(fn: str, st: int) -> None:
    if st in (PA_ERR_NO_BLOCKS, PA_ERR_NO_SEQUENCE):
        raise BlockManagerError(fn, st)
    if st < 0:
        raise PaError(fn, st)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int):
        self._lib = _lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("pa_bm_create failed (non-positive sizes or out of memory)")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def add_sequence(self, tokens) -> tuple[int, int]:
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        sid, cached = ctypes.c_int64(), ctypes.c_int32()
        st = self._lib.pa_bm_add_sequence(self._h, t.ctypes.data if t.size else None, int(t.size),
                                          ctypes.byref(sid), ctypes.byref(cached))
        _check("pa_bm_add_sequence", st)
        return int(sid.value), int(cached.value)

    def append(self, sid: int, token: int) -> int:
        slot = ctypes.c_int64()
        _check("pa_bm_append", self._lib.pa_bm_append(self._h, int(sid), int(token), ctypes.byref(slot)))
        return int(slot.value)

    def append_batch(self, sids, tokens) -> np.ndarray:
        """One decode step: token tokens[i] onto sequence sids[i]; returns the
        slots (int64, the step's slot_mapping).  All or nothing."""
        ids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        if ids.shape != tok.shape or ids.ndim != 1:
            raise ValueError("sids and tokens must be 1-D of equal length")
        slots = np.empty(max(ids.size, 1), dtype=np.int64)
        n = int(ids.size)
        _check("pa_bm_append_batch", self._lib.pa_bm_append_batch(
            self._h, ids.ctypes.data if n else None, tok.ctypes.data if n else None, n,
            slots.ctypes.data if n else None))
        return slots[:n]

    def free_sequence(self, sid: int) -> None:
        _check("pa_bm_free_sequence", self._lib.pa_bm_free_sequence(self._h, int(sid)))

    def length(self, sid: int) -> int:
        n = int(self._lib.pa_bm_length(self._h, int(sid)))
        _check("pa_bm_length", min(n, 0))
        return n

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def block_table(self, sid: int) -> list:
        nb = ctypes.c_int32()
        st = self._lib.pa_bm_block_table(self._h, int(sid), None, 0, ctypes.byref(nb))
        if st not in (0, -2):
            _check("pa_bm_block_table", st)
        out = np.empty(max(nb.value, 1), dtype=np.int32)
        _check("pa_bm_block_table", self._lib.pa_bm_block_table(self._h, int(sid), out.ctypes.data, int(out.size),
                                                                ctypes.byref(nb)))
        return out[:nb.value].tolist()

    def slots(self, sid: int, start: int, count: int) -> list:
        out = np.empty(max(int(count), 1), dtype=np.int64)
        _check("pa_bm_slots", self._lib.pa_bm_slots(self._h, int(sid), int(start), int(count), out.ctypes.data))
        return out[:int(count)].tolist()

    def fill_tables(self, sids, max_blocks_per_seq: int, fill: int = 0):
        """(block_tables int32 [B, W], context_lens int32 [B]) on the host."""
        ids = np.ascontiguousarray(np.asarray(sids, dtype=np.int64))
        B, W = int(ids.size), int(max_blocks_per_seq)
        tables = np.empty((B, W), dtype=np.int32)
        lens = np.empty(B, dtype=np.int32)
        _check("pa_bm_fill_tables", self._lib.pa_bm_fill_tables(
            self._h, ids.ctypes.data if B else None, B, W, int(fill), tables.ctypes.data if B else None,
            lens.ctypes.data if B else None))
        return tables, lens
