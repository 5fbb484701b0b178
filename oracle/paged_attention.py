"""Plain fp64 CPU oracle for paged decode attention and the new-token cache write.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (``paged_kv_cache_438_amd``) never imports it, and it imports nothing
from the product path: the two share no code.

What is computed, and where the pages define it:

* A sequence's keys and values live in fixed-size blocks of a pool; a
  per-sequence table lists, in logical order, which physical block holds
  each stretch of ``block_size`` tokens ("IO-5 vLLM Paged Attention",
  section 2 "Paged Attention idea" and section 3 "KV Cache Paging
  structure"; "Efficient Memory Management for LLM Serving with
  PagedAttention (vLLM) paper summary", key feature 1 "KV cache blocking"
  and key feature 3, the page-table analogy).
* The number of blocks a sequence of ``L`` tokens occupies is the ceiling of
  L / block_size ("vLLM's efficiency secret: PagedAttention and dynamic
  memory management", section "Dynamic memory management", the
  BlockSpaceManager example).
* Attention is the ordinary softmax(q K^T * scale) V, where K and V are the
  sequence's pages concatenated in table order ("IO-5 vLLM Paged
  Attention", section 4 "Attention computation").  Paging does not change
  the attention result (same page, "5 common misconceptions", the first
  two), so the oracle is that definition written out: gather, concatenate,
  textbook softmax, weighted sum.

Readings where the pages are silent (each is also listed in the design
notes):

* R1  Only the first L rows of the concatenation belong to the sequence;
      rows past L in the last block and blocks past ceil(L/bs) are never
      read.  (Waste is max length minus actual length: "IO-5 vLLM Paged
      Attention", section 1 "Existing KV cache problem".)
* R2  Grouped query heads: query head h reads KV head h // (Hq / Hkv).
* R3  L = 0 gives an all-zero output and no cache write.
* R4  ``context_lens`` already counts the new token, which sits at logical
      position L-1; the cache write copies its K/V rows there.
* R5  ``scale`` is a float32 value; the oracle widens that same value.
* R6  Inputs are widened exactly to fp64 (bf16 from its raw bits).

Parity: every function here is pinned by tests in ``tests/test_oracle_pins.py``
(brute force on tiny inputs, closed forms, a hand-worked fixture on the
pages' page-table example, placement/sharing/grouping invariances, the
partition merge identity).  No function is left unpinned.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------- widening
def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to fp64 (R6).  bf16 arrives as raw
    uint16 bits: its value is the fp32 number whose upper 16 bits they are."""
    if dtype in ("f32", "f16"):
        return np.asarray(x).astype(np.float64)
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- paging
def blocks_needed(seq_len: int, block_size: int) -> int:
    """Ceiling division of tokens by page size ("vLLM's efficiency secret",
    section "Dynamic memory management": 3200 tokens at 512 per page need
    7 pages)."""
    return (seq_len + block_size - 1) // block_size


def gather_kv(pool: np.ndarray, table_row: Sequence[int], seq_len: int,
              kv_head: int, block_size: int) -> np.ndarray:
    """K (or V) of one sequence and one KV head as a contiguous [L][d] array:
    the sequence's pages concatenated in table order ("IO-5 vLLM Paged
    Attention", section 4), cut to its first L rows (R1)."""
    nb = blocks_needed(seq_len, block_size)
    pages = [pool[int(table_row[i]), kv_head] for i in range(nb)]   # each [bs][d]
    if not pages:
        return pool[:0, kv_head, 0]   # shape [0][d]
    return np.concatenate(pages, axis=0)[:seq_len]


# ---------------------------------------------------------------- attention
def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q K^T * scale) V for one query vector, in fp64 ("IO-5 vLLM
    Paged Attention", section 4).  Subtracting the maximum score before
    exponentiating leaves the softmax unchanged and keeps exp finite."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)        # R3
    z = (K @ q) * scale
    w = np.exp(z - z.max())
    p = w / w.sum()
    return p @ V


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, scale, block_size: int,
           dtype: str, pairs: Optional[Iterable[Tuple[int, int]]] = None) -> np.ndarray:
    """Paged decode attention for every (sequence, query head), or only for
    the listed ``pairs``.

    q: [B][Hq][d]; pools: [NB][Hkv][bs][d]; block_tables: [B][MB];
    context_lens: [B].  Returns fp64 [B][Hq][d] (entries not in ``pairs``
    are NaN).
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv                                     # R2
    scale64 = float(np.float32(scale))               # R5
    out = np.full((B, Hq, d), np.nan, dtype=np.float64)
    if pairs is None:
        pairs = [(s, h) for s in range(B) for h in range(Hq)]
    by_seq_head = {}
    for s, h in pairs:
        by_seq_head.setdefault((s, h // G), []).append(h)
    for (s, g), heads in sorted(by_seq_head.items()):
        L = int(context_lens[s])
        K = widen(gather_kv(k_pool, block_tables[s], L, g, block_size), dtype)
        V = widen(gather_kv(v_pool, block_tables[s], L, g, block_size), dtype)
        for h in heads:
            out[s, h] = softmax_attention(widen(q[s, h], dtype), K, V, scale64)
    return out


def decode_partitioned(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                       block_tables: np.ndarray, context_lens: np.ndarray, scale,
                       block_size: int, dtype: str, partition_size: int) -> np.ndarray:
    """The same attention computed partition by partition and merged
    (test-only form of the split-K path).  Each partition p of a sequence
    covers tokens [p*P, min((p+1)*P, L)) and yields its own maximum m_p,
    sum l_p = sum exp(z - m_p) and unnormalised a_p = sum exp(z - m_p) v.
    With M = max m_p the merged output is
    sum_p a_p exp(m_p - M) / sum_p l_p exp(m_p - M), which equals the
    softmax over all tokens exactly (the exp(m_p - M) factors restore the
    common reference point)."""
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    out = np.zeros((B, Hq, d), dtype=np.float64)
    for s in range(B):
        L = int(context_lens[s])
        if L == 0:
            continue
        for g in range(Hkv):
            K = widen(gather_kv(k_pool, block_tables[s], L, g, block_size), dtype)
            V = widen(gather_kv(v_pool, block_tables[s], L, g, block_size), dtype)
            for h in range(g * G, (g + 1) * G):
                qh = widen(q[s, h], dtype)
                parts = []
                for lo in range(0, L, partition_size):
                    hi = min(lo + partition_size, L)
                    z = (K[lo:hi] @ qh) * scale64
                    m = z.max()
                    w = np.exp(z - m)
                    parts.append((m, w.sum(), w @ V[lo:hi]))
                M = max(p[0] for p in parts)
                num = sum(a * math.exp(m - M) for m, _, a in parts)
                den = sum(l * math.exp(m - M) for m, l, _ in parts)
                out[s, h] = num / den
    return out


# ---------------------------------------------------------------- cache write
def cache_write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                v_new: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Store each sequence's newest token (logical position L-1, R4) into the
    row of the page that the table names for it: page table[s][(L-1) // bs],
    row (L-1) % bs, every KV head.  The copy is bytewise; every other byte of
    both pools is unchanged.  Returns new pools (inputs are not modified)."""
    kp, vp = k_pool.copy(), v_pool.copy()
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        if L < 1:
            continue                                  # R3
        pos = L - 1
        blk = int(block_tables[s][pos // block_size])
        row = pos % block_size
        kp[blk, :, row, :] = k_new[s]
        vp[blk, :, row, :] = v_new[s]
    return kp, vp


def cache_write_contiguous(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray,
                           v_new: np.ndarray, context_lens: np.ndarray
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """The same write for the pre-paging layout, where each request owns one
    contiguous region of max_len rows per KV head ("IO-5 vLLM Paged
    Attention", section 1): the newest token (position L-1, R4) goes to row
    L-1 of k_cache[s][g] and v_cache[s][g], [B][Hkv][max_len][d], every KV
    head.  L = 0 writes nothing (R3); a length past max_len does not fit and
    writes nothing either.  Bytewise; returns new caches."""
    kc, vc = k_cache.copy(), v_cache.copy()
    max_len = k_cache.shape[2]
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        if L < 1 or L > max_len:
            continue
        kc[s, :, L - 1, :] = k_new[s]
        vc[s, :, L - 1, :] = v_new[s]
    return kc, vc


def contiguous_attention(q: np.ndarray, K_seqs: List[np.ndarray], V_seqs: List[np.ndarray],
                         scale, dtype: str, num_kv_heads: int) -> np.ndarray:
    """Attention over per-sequence contiguous K/V ([L][Hkv][d] each), the
    pre-paging layout where each request owns one contiguous buffer ("IO-5
    vLLM Paged Attention", section 1).  Used to check that paging changes
    nothing."""
    B, Hq, d = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((B, Hq, d), dtype=np.float64)
    scale64 = float(np.float32(scale))
    for s in range(B):
        for h in range(Hq):
            K = widen(K_seqs[s][:, h // G, :], dtype)
            V = widen(V_seqs[s][:, h // G, :], dtype)
            out[s, h] = softmax_attention(widen(q[s, h], dtype), K, V, scale64)
    return out
