"""Plain CPU oracle of the block moves around decode: whole-block copies
inside the pools and block swaps between the GPU pool and a CPU pool.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; it shares no
code with the product path.

* Block-level sharing lets several requests name the same physical block
  ("Efficient Memory Management for LLM Serving with PagedAttention (vLLM)
  paper summary", key feature 2, "KV cache sharing").  A request about to
  write into a partly filled block that others share first gets a private
  copy of it (reading R17, copy-on-write): every byte of the source block,
  in every KV head, of both the key and the value pool, goes to the
  destination block.
* The block manager also keeps CPU blocks ("vLLM's efficiency secret:
  PagedAttention and dynamic memory management", section "Dynamic memory
  management", num_cpu_blocks); swapping moves a block's bytes, both pools,
  between a GPU block and a CPU block (reading R19).

Both are byte moves, so the oracle is the definition: for each (source,
destination) pair, destination := source, bit for bit; nothing else changes.
Pins: tests/golden/block_ops_example.json (a hand-written 4-block fixture
with its expected pools), the swap round trip, and decode through a copied
block equalling decode through the original (tests/test_oracle_pins.py).
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def _pair_list(pairs) -> list:
    return [(int(a), int(b)) for a, b in np.asarray(pairs, dtype=np.int64).reshape(-1, 2)]


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray,
                pairs: Iterable[Tuple[int, int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of both pools ([NB][Hkv][bs][d]) in which block ``dst`` holds
    the bytes of block ``src`` for every pair.  A pair naming a block outside
    [0, NB), or with src == dst, moves nothing (the library skips such
    pairs).  Destinations must be distinct and must not be the source of
    another pair: then the order of the pairs does not matter."""
    NB = k_pool.shape[0]
    assert v_pool.shape == k_pool.shape
    moves = [(s, d) for s, d in _pair_list(pairs) if 0 <= s < NB and 0 <= d < NB and s != d]
    dsts = [d for _, d in moves]
    if len(set(dsts)) != len(dsts) or set(dsts) & {s for s, _ in moves}:
        raise ValueError("destinations must be distinct and must not be sources")
    kp, vp = k_pool.copy(), v_pool.copy()
    for s, d in moves:
        kp[d] = k_pool[s]
        vp[d] = v_pool[s]
    return kp, vp


def swap_blocks(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray, src_v: np.ndarray,
                pairs: Iterable[Tuple[int, int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the destination pools in which block ``dst`` holds the
    bytes of source block ``src`` for every (src, dst) pair; one pool pair
    is the GPU pool and the other the CPU pool, in either direction.  Pairs
    outside either pool are an error (the library refuses the call)."""
    assert dst_k.shape[1:] == src_k.shape[1:] and dst_v.shape == dst_k.shape
    assert src_v.shape == src_k.shape
    moves = _pair_list(pairs)
    for s, d in moves:
        if not (0 <= s < src_k.shape[0] and 0 <= d < dst_k.shape[0]):
            raise ValueError(f"pair ({s}, {d}) outside the pools")
    if len({d for _, d in moves}) != len(moves):
        raise ValueError("destinations must be distinct")
    dk, dv = dst_k.copy(), dst_v.copy()
    for s, d in moves:
        dk[d] = src_k[s]
        dv[d] = src_v[s]
    return dk, dv
