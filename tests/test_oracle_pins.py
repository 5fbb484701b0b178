"""CPU tests: the fp64 oracle against its pins, and planted mistakes in the
oracle caught by those pins."""
import math

import numpy as np
import pytest

import oracle.paged_attention as PA
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(PA)


# ------------------------------------------------------------ planted mistakes
# Each mutant is a plausible slip in the oracle.  It is planted on the CPU by
# patching the oracle module; at least one pin must then fail.

def _gather_ignoring_table(pool, table_row, seq_len, kv_head, block_size):
    nb = PA.blocks_needed(seq_len, block_size)
    pages = [pool[i, kv_head] for i in range(nb)]          # logical id used as physical
    if not pages:
        return pool[:0, kv_head, 0]
    return np.concatenate(pages, axis=0)[:seq_len]


def _gather_keeping_tail(pool, table_row, seq_len, kv_head, block_size):
    nb = PA.blocks_needed(seq_len, block_size)
    pages = [pool[int(table_row[i]), kv_head] for i in range(nb)]
    if not pages:
        return pool[:0, kv_head, 0]
    return np.concatenate(pages, axis=0)                   # not cut to L


def _softmax_no_scale(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    z = K @ q
    w = np.exp(z - z.max())
    return (w / w.sum()) @ V


def _softmax_no_max(q, K, V, scale):
    if K.shape[0] == 0:
        return np.zeros(V.shape[1])
    w = np.exp((K @ q) * scale)
    return (w / w.sum()) @ V


def _widen_bad_bf16(x, dtype):
    if dtype == "bf16":
        b = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
        return b.view(np.float32).astype(np.float64)
    return np.asarray(x).astype(np.float64)


def _cache_write_at_L(k_pool, v_pool, k_new, v_new, block_tables, context_lens, block_size):
    kp, vp = k_pool.copy(), v_pool.copy()
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        if L < 1:
            continue
        pos = L                                               # off by one
        blk = int(block_tables[s][min(pos // block_size, block_tables.shape[1] - 1)])
        kp[blk, :, pos % block_size, :] = k_new[s]
        vp[blk, :, pos % block_size, :] = v_new[s]
    return kp, vp


def _cache_write_contiguous_at_L(k_cache, v_cache, k_new, v_new, context_lens):
    kc, vc = k_cache.copy(), v_cache.copy()
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        if L < 1 or L >= k_cache.shape[2]:
            continue
        kc[s, :, L, :] = k_new[s]                             # off by one
        vc[s, :, L, :] = v_new[s]
    return kc, vc


def _decode_gqa_modulo(q, k_pool, v_pool, block_tables, context_lens, scale, block_size,
                       dtype, pairs=None):
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    out = np.zeros((B, Hq, d))
    for s in range(B):
        L = int(context_lens[s])
        for h in range(Hq):
            g = h % Hkv                                       # wrong grouping
            K = PA.widen(PA.gather_kv(k_pool, block_tables[s], L, g, block_size), dtype)
            V = PA.widen(PA.gather_kv(v_pool, block_tables[s], L, g, block_size), dtype)
            out[s, h] = PA.softmax_attention(PA.widen(q[s, h], dtype), K, V,
                                             float(np.float32(scale)))
    return out


def _decode_kv_swapped(q, k_pool, v_pool, *a, **kw):
    return _ORIG_DECODE(q, v_pool, k_pool, *a, **kw)


_ORIG_DECODE = PA.decode

MUTANTS = {
    "table_ignored": ("gather_kv", _gather_ignoring_table),
    "tail_rows_kept": ("gather_kv", _gather_keeping_tail),
    "block_count_floored": ("blocks_needed", lambda L, bs: L // bs),
    "scale_dropped": ("softmax_attention", _softmax_no_scale),
    "max_not_subtracted": ("softmax_attention", _softmax_no_max),
    "bf16_widen_shift": ("widen", _widen_bad_bf16),
    "cache_write_at_L": ("cache_write", _cache_write_at_L),
    "contiguous_write_at_L": ("cache_write_contiguous", _cache_write_contiguous_at_L),
    "gqa_modulo_mapping": ("decode", _decode_gqa_modulo),
    "k_v_swapped": ("decode", _decode_kv_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(PA, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(PA)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"planted mistake {name!r} passed every pin"
