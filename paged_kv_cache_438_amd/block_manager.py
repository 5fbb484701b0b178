"""Python handle on the library's host-side block manager
(include/pa_block_manager.h).  Argument marshalling only: the bookkeeping is
the C++ code in libpa.so."""
from __future__ import annotations

import ctypes
from typing import List, Optional, Tuple

import numpy as np

from ._binding import PaError, last_error, load

PA_ERR_OUT_OF_BLOCKS = 6


class OutOfBlocks(PaError):
    """Too few free blocks; the manager is unchanged."""


def _check(st: int, func: str) -> None:
    if st != 0:
        cls = OutOfBlocks if st == PA_ERR_OUT_OF_BLOCKS else PaError
        raise cls(st, func, last_error())


class BlockManager:
    """Free lists, reference counts, copy-on-write and swap bookkeeping for a
    pool of ``num_gpu_blocks`` GPU blocks and ``num_cpu_blocks`` CPU blocks of
    ``block_size`` tokens."""

    def __init__(self, block_size: int, num_gpu_blocks: int, num_cpu_blocks: int = 0):
        self._lib = load()
        h = ctypes.c_void_p()
        _check(self._lib.pa_bm_create(block_size, num_gpu_blocks, num_cpu_blocks, ctypes.byref(h)),
               "pa_bm_create")
        self._h = h
        self.block_size = block_size
        self.num_gpu_blocks = num_gpu_blocks
        self.num_cpu_blocks = num_cpu_blocks

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def can_allocate(self, num_tokens: int) -> bool:
        r = self._lib.pa_bm_can_allocate(self._h, num_tokens)
        if r < 0:
            _check(-r, "pa_bm_can_allocate")
        return bool(r)

    def allocate(self, seq_id: int, num_tokens: int) -> None:
        _check(self._lib.pa_bm_allocate(self._h, seq_id, num_tokens), "pa_bm_allocate")

    def append_slot(self, seq_id: int) -> Tuple[int, int, Optional[Tuple[int, int]]]:
        """Room for one more token: (block, row) of the new token, and the
        (source, destination) blocks to copy if a shared block was replaced."""
        b, r, cs, cd = (ctypes.c_int32() for _ in range(4))
        _check(self._lib.pa_bm_append_slot(self._h, seq_id, ctypes.byref(b), ctypes.byref(r),
                                           ctypes.byref(cs), ctypes.byref(cd)), "pa_bm_append_slot")
        return b.value, r.value, ((cs.value, cd.value) if cs.value >= 0 else None)

    def fork(self, parent_id: int, child_id: int) -> None:
        _check(self._lib.pa_bm_fork(self._h, parent_id, child_id), "pa_bm_fork")

    def free(self, seq_id: int) -> None:
        _check(self._lib.pa_bm_free(self._h, seq_id), "pa_bm_free")

    def _swap(self, fn, seq_id: int) -> List[Tuple[int, int]]:
        _, nb, _ = self.seq_info(seq_id)
        pairs = np.zeros((max(nb, 1), 2), dtype=np.int32)
        n = ctypes.c_int(0)
        _check(getattr(self._lib, fn)(self._h, seq_id, pairs.ctypes.data, nb, ctypes.byref(n)), fn)
        return [(int(a), int(b)) for a, b in pairs[:n.value]]

    def swap_out(self, seq_id: int) -> List[Tuple[int, int]]:
        return self._swap("pa_bm_swap_out", seq_id)

    def swap_in(self, seq_id: int) -> List[Tuple[int, int]]:
        return self._swap("pa_bm_swap_in", seq_id)

    def num_free(self, on_cpu: bool = False) -> int:
        r = self._lib.pa_bm_num_free_blocks(self._h, int(on_cpu))
        if r < 0:
            _check(-r, "pa_bm_num_free_blocks")
        return r

    def usage_ratio(self) -> float:
        return float(self._lib.pa_bm_usage_ratio(self._h))

    def seq_info(self, seq_id: int) -> Tuple[int, int, bool]:
        """(tokens, blocks, on_cpu) of a sequence."""
        t, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check(self._lib.pa_bm_seq_info(self._h, seq_id, ctypes.byref(t), ctypes.byref(b),
                                        ctypes.byref(c)), "pa_bm_seq_info")
        return t.value, b.value, bool(c.value)

    def refcount(self, block: int, on_cpu: bool = False) -> int:
        r = self._lib.pa_bm_refcount(self._h, block, int(on_cpu))
        if r < 0:
            _check(-r, "pa_bm_refcount")
        return r

    def fill_batch(self, seq_ids, max_blocks_per_seq: int) -> Tuple[np.ndarray, np.ndarray]:
        """Host block tables [n][max_blocks_per_seq] (padding -1) and lengths [n]."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
        n = ids.shape[0]
        tables = np.empty((n, max_blocks_per_seq), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        _check(self._lib.pa_bm_fill_batch(self._h, ids.ctypes.data, n, tables.ctypes.data,
                                          max_blocks_per_seq, lens.ctypes.data),
               "pa_bm_fill_batch")
        return tables, lens

    def prefix_groups(self, seq_ids) -> Tuple[np.ndarray, np.ndarray, int]:
        """(seq_group [n], group_prefix_len [groups], max_group_size) for
        pa_decode_shared_prefix."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
        n = ids.shape[0]
        group = np.empty(max(n, 1), dtype=np.int32)
        prefix = np.empty(max(n // 2, 1), dtype=np.int32)
        ng, mg = ctypes.c_int(), ctypes.c_int()
        _check(self._lib.pa_bm_prefix_groups(self._h, ids.ctypes.data, n, group.ctypes.data,
                                             prefix.ctypes.data, ctypes.byref(ng),
                                             ctypes.byref(mg)), "pa_bm_prefix_groups")
        return group[:n].copy(), prefix[:ng.value].copy(), mg.value
