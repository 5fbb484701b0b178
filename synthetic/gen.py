"""Seeded synthetic inputs for paged decode attention.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the attention arithmetic: it draws random numbers, rounds them
to the storage dtype and places each sequence's logical K/V rows into
physical blocks of a pool, recording the block table that maps logical block
i of sequence s to its physical block ("IO-5 vLLM Paged Attention",
section 2 "Paged Attention idea": a request lists the pages it uses, such as
pages 1, 5 and 9; section 3: the cache is a list of pages and each sequence
owns a list of page indices).

Draw order (fixed, so a seed reproduces the same bytes):
  1. lengths, 2. block permutation, 3. Q, 4. per sequence its logical K then
  V.  Shared-prefix workloads go group by group: the group's prompt K then V,
  then each member's suffix K then V.

Values are drawn in fp32 and rounded to nearest-even into the storage dtype.
bf16 is stored as raw uint16 bits (numpy has no bf16 type).

Blocks are assigned by taking ids from the permutation in the same order as
the draws: sequence by sequence, each in logical order; for shared-prefix
workloads a group's prompt blocks come first, then each member's suffix
blocks, and every member's table lists the same prompt blocks.  Unused blocks and the
rows of a last block past the sequence's length are filled with NaN when
``poison`` is set, so that any read of them shows up in the output.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from .configs import Workload

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
NAN_BITS = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits.
    Inputs are finite (normal draws)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Case:
    workload: Workload
    seed: int
    q: np.ndarray                 # [B][Hq][d] storage dtype
    k_pool: np.ndarray            # [NB][Hkv][bs][d] storage dtype
    v_pool: np.ndarray
    block_tables: np.ndarray      # int32 [B][MB], padding -1
    context_lens: np.ndarray      # int32 [B]
    k_new: np.ndarray             # [B][Hkv][d]: logical token L-1 of each sequence
    v_new: np.ndarray
    scale: np.float32
    num_blocks: int
    unique_blocks: int            # physical blocks in use
    new_slots: np.ndarray         # int64 [B][2]: (block id, row) holding token L-1; -1 if L=0
    logical_k: Optional[List[np.ndarray]] = None   # per sequence [L][Hkv][d]
    logical_v: Optional[List[np.ndarray]] = None
    shared_groups: Optional[np.ndarray] = None     # [groups][group_size] sequence ids
    prompt_blocks: int = 0

    @property
    def dtype(self) -> str:
        return self.workload.dtype

    @property
    def block_size(self) -> int:
        return self.workload.block_size

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.q, self.k_pool, self.v_pool, self.block_tables, self.context_lens,
                  self.k_new, self.v_new):
            h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
        return h.hexdigest()

    def pools_with_new_slots_poisoned(self) -> Tuple[np.ndarray, np.ndarray]:
        """Copies of the pools in which the row of each sequence's newest token
        holds NaN: the state just before that token's K/V are written."""
        kp, vp = self.k_pool.copy(), self.v_pool.copy()
        nan = NAN_BITS[self.dtype]
        for b, r in self.new_slots:
            if b >= 0:
                kp[b, :, r, :] = nan
                vp[b, :, r, :] = nan
        return kp, vp


def draw_lengths(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.length_kind == "fixed":
        assert len(w.lengths) == w.num_seqs
        return np.array(w.lengths, dtype=np.int64)
    if w.length_kind == "uniform":
        return rng.integers(w.length_lo, w.length_hi, size=w.num_seqs, endpoint=True)
    if w.length_kind == "lognormal":
        x = rng.normal(np.log(w.lognormal_median), w.lognormal_sigma, size=w.num_seqs)
        return np.clip(np.rint(np.exp(x)), w.length_lo, w.length_hi).astype(np.int64)
    if w.length_kind == "shared_prefix":
        assert w.groups * w.group_size == w.num_seqs
        assert w.prompt_len % w.block_size == 0
        suffix = rng.integers(w.length_lo, w.length_hi, size=w.num_seqs, endpoint=True)
        return w.prompt_len + suffix
    raise ValueError(w.length_kind)


def _normal(rng, shape, std) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _place(pool: np.ndarray, ids: np.ndarray, rows: np.ndarray, bs: int, nan) -> None:
    """Write logical rows [n][Hkv][d] into blocks ``ids`` (logical order)."""
    n, hkv, d = rows.shape
    nb = len(ids)
    pad = nb * bs - n
    if pad:
        rows = np.concatenate([rows, np.full((pad, hkv, d), nan, dtype=rows.dtype)], axis=0)
    pool[ids] = rows.reshape(nb, bs, hkv, d).transpose(0, 2, 1, 3)


def make_case(w: Workload, seed: Optional[int] = None, poison: bool = True,
              keep_logical: bool = False) -> Case:
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, bs = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    st = STORAGE[w.dtype]
    nan = NAN_BITS[w.dtype]

    lens = draw_lengths(w, rng)                                     # 1
    shared = w.length_kind == "shared_prefix"
    if shared:
        pb = w.prompt_len // bs
        suffix_blocks = [ceil_div(int(L) - w.prompt_len, bs) for L in lens]
        unique = w.groups * pb + sum(suffix_blocks)
    else:
        pb = 0
        unique = sum(ceil_div(int(L), bs) for L in lens)
    NB = w.num_blocks if w.num_blocks is not None else w.pool_factor * unique
    assert NB >= unique
    MB = w.max_blocks_per_seq
    assert int(max(ceil_div(int(L), bs) for L in lens)) <= MB
    perm = rng.permutation(NB)                                      # 2
    q = to_storage(_normal(rng, (B, Hq, d), w.q_std), w.dtype)      # 3

    fill = nan if poison else st(0)
    k_pool = np.full((NB, Hkv, bs, d), fill, dtype=st)
    v_pool = np.full((NB, Hkv, bs, d), fill, dtype=st)
    tables = np.full((B, MB), -1, dtype=np.int32)
    k_new = np.zeros((B, Hkv, d), dtype=st)
    v_new = np.zeros((B, Hkv, d), dtype=st)
    new_slots = np.full((B, 2), -1, dtype=np.int64)
    lk: Optional[list] = [None] * B if keep_logical else None
    lv: Optional[list] = [None] * B if keep_logical else None
    nxt = 0

    def take(n):
        nonlocal nxt
        ids = perm[nxt:nxt + n]
        nxt += n
        return ids

    def finish_seq(s, ids, K, V):
        L = int(lens[s])
        tables[s, :len(ids)] = ids
        if L >= 1:
            k_new[s] = K[L - 1]
            v_new[s] = V[L - 1]
            new_slots[s] = (ids[(L - 1) // bs], (L - 1) % bs)
        if keep_logical:
            lk[s], lv[s] = K, V

    groups_arr = None
    if shared:
        groups_arr = np.arange(B).reshape(w.groups, w.group_size)
        for gi in range(w.groups):
            Kp = to_storage(_normal(rng, (w.prompt_len, Hkv, d), w.kv_std), w.dtype)  # 4
            Vp = to_storage(_normal(rng, (w.prompt_len, Hkv, d), w.kv_std), w.dtype)
            pids = take(pb)
            _place(k_pool, pids, Kp, bs, nan)
            _place(v_pool, pids, Vp, bs, nan)
            for s in groups_arr[gi]:
                n = int(lens[s]) - w.prompt_len
                Ks = to_storage(_normal(rng, (n, Hkv, d), w.kv_std), w.dtype)       # 5
                Vs = to_storage(_normal(rng, (n, Hkv, d), w.kv_std), w.dtype)
                sids = take(ceil_div(n, bs))
                _place(k_pool, sids, Ks, bs, nan)
                _place(v_pool, sids, Vs, bs, nan)
                finish_seq(s, np.concatenate([pids, sids]),
                           np.concatenate([Kp, Ks]), np.concatenate([Vp, Vs]))
    else:
        for s in range(B):
            L = int(lens[s])
            K = to_storage(_normal(rng, (L, Hkv, d), w.kv_std), w.dtype)            # 5
            V = to_storage(_normal(rng, (L, Hkv, d), w.kv_std), w.dtype)
            ids = take(ceil_div(L, bs))
            if L:
                _place(k_pool, ids, K, bs, nan)
                _place(v_pool, ids, V, bs, nan)
            finish_seq(s, ids, K, V)

    scale = np.float32(1.0 / np.sqrt(np.float32(d)))
    return Case(workload=w, seed=seed, q=q, k_pool=k_pool, v_pool=v_pool,
                block_tables=tables, context_lens=lens.astype(np.int32),
                k_new=k_new, v_new=v_new, scale=scale, num_blocks=NB,
                unique_blocks=unique, new_slots=new_slots, logical_k=lk, logical_v=lv,
                shared_groups=groups_arr, prompt_blocks=pb)


def contiguous_cache(case: Case, max_len: Optional[int] = None, poison: bool = True,
                     device=None):
    """The case's K and V laid out as a contiguous cache instead of a pool:
    [B][Hkv][max_len][d] each, row t of sequence s's region holding its
    logical token t (the generator's own draws, kept by ``make_case(...,
    keep_logical=True)``).  Rows past a sequence's length hold NaN (zero
    without ``poison``).  ``max_len`` defaults to the longest length.

    Host arrays in the storage dtype (uint16 bits for bf16); with ``device``,
    torch tensors built there sequence by sequence (no host copy of the
    whole cache)."""
    if case.logical_k is None:
        raise ValueError("contiguous_cache needs make_case(..., keep_logical=True)")
    w = case.workload
    lens = case.context_lens.astype(np.int64)
    if max_len is None:
        max_len = max(1, int(lens.max()))
    if int(lens.max()) > max_len:
        raise ValueError(f"a sequence of {int(lens.max())} tokens does not fit max_len {max_len}")
    st = STORAGE[w.dtype]
    fill = NAN_BITS[w.dtype] if poison else st(0)
    shape = (w.num_seqs, w.num_kv_heads, max_len, w.head_dim)
    if device is None:
        kc = np.full(shape, fill, dtype=st)
        vc = np.full(shape, fill, dtype=st)
    else:
        import torch
        # bf16 travels as its int16 bit pattern and is reinterpreted at the end.
        bits = {"f32": (np.float32, torch.float32), "f16": (np.float16, torch.float16),
                "bf16": (np.int16, torch.int16)}[w.dtype]
        fill_t = np.array([fill], dtype=st).view(bits[0])[0].item()
        kc = torch.full(shape, fill_t, dtype=bits[1], device=device)
        vc = torch.full(shape, fill_t, dtype=bits[1], device=device)
    for s in range(w.num_seqs):
        L = int(lens[s])
        if not L:
            continue
        for cache, rows in ((kc, case.logical_k[s]), (vc, case.logical_v[s])):
            region = np.ascontiguousarray(rows.transpose(1, 0, 2))
            if device is None:
                cache[s, :, :L] = region
            else:
                cache[s, :, :L].copy_(torch.from_numpy(region.view(bits[0])))
    if device is not None and w.dtype == "bf16":
        kc, vc = kc.view(torch.bfloat16), vc.view(torch.bfloat16)
    return kc, vc


def kv_token_count(case: Case) -> int:
    """Logical KV tokens attended by one decode step (all heads of a token
    count once)."""
    return int(case.context_lens.astype(np.int64).sum())


def algorithmic_bytes(case: Case, unique: bool = False, tables: bool = True) -> int:
    """Bytes a paged decode step must move: K and V over valid rows, Q in,
    output out, block-table entries in use and lengths.  With ``unique``, a
    shared prompt's rows are counted once per group instead of once per
    sequence; without ``tables``, no table entries (a contiguous cache)."""
    w = case.workload
    e = w.elem_bytes
    lens = case.context_lens.astype(np.int64)
    tokens = int(lens.sum())
    if unique and case.shared_groups is not None:
        tokens -= (w.group_size - 1) * w.groups * w.prompt_len
    kv = tokens * 2 * w.num_kv_heads * w.head_dim * e
    qo = 2 * w.num_seqs * w.num_heads * w.head_dim * e
    nb = int(sum(ceil_div(int(L), w.block_size) for L in lens)) if tables else 0
    meta = 4 * (nb + w.num_seqs)
    return kv + qo + meta
