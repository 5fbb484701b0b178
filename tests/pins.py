"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError if
the oracle disagrees with something the pages or the mathematics fix.  The
tests call them with the real oracle, and ``test_oracle_pins`` also calls
them with deliberately broken copies of it, to show that a plausible mistake
(a wrong index, a dropped factor, a missing cut) fails at least one pin.
"""
from __future__ import annotations

import json
import math
import pathlib
import struct

import numpy as np

from synthetic import (GQA70B, LLAMA7B, LONG_BS512, SHARED_PREFIX, TINY, NAN_BITS,
                       contiguous_cache, make_case, small_variant, to_storage)

GOLDEN = pathlib.Path(__file__).parent / "golden"


# --------------------------------------------------------------- fixtures
def load_page_table_example():
    """The hand-worked fixture built on the pages' page-table example
    (request A -> pages 1, 5, 9; request B -> pages 2, 3)."""
    fx = json.loads((GOLDEN / "page_table_example.json").read_text())
    logs = {"L2": math.log(2), "L4": math.log(4), "L3": math.log(3), "L9": math.log(9)}

    def val(x):
        if isinstance(x, str):
            if x.startswith("2*"):
                return 2 * logs[x[2:]]
            return logs[x]
        return float(x)

    bs, d, NB = fx["block_size"], fx["head_dim"], fx["num_blocks"]
    kp = np.full((NB, 1, bs, d), np.nan, dtype=np.float32)
    vp = np.full((NB, 1, bs, d), np.nan, dtype=np.float32)
    for pool, pages in ((kp, fx["k_pages"]), (vp, fx["v_pages"])):
        for pid, rows in pages.items():
            for r, row in enumerate(rows):
                if row != "NaN":
                    pool[int(pid), 0, r] = [val(x) for x in row]
    names = ["A", "B"]
    MB = max(len(fx["block_tables"][n]) for n in names)
    tables = np.full((2, MB), -1, dtype=np.int32)
    for i, n in enumerate(names):
        t = fx["block_tables"][n]
        tables[i, :len(t)] = t
    lens = np.array([fx["context_lens"][n] for n in names], dtype=np.int32)
    q = np.array([[fx["q"][n]] for n in names], dtype=np.float32)
    expected = np.array([[fx["expected_out"][n]] for n in names])
    slots = [tuple(fx["cache_write"]["expected_slots"][n]) for n in names]
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=lens, scale=np.float32(fx["scale"]),
                bs=bs, expected=expected, tol=fx["tolerance"], slots=slots)


def pin_page_table_example(O):
    fx = load_page_table_example()
    out = O.decode(fx["q"], fx["kp"], fx["vp"], fx["tables"], fx["lens"], fx["scale"],
                   fx["bs"], "f32")
    assert np.all(np.isfinite(out)), out
    assert np.max(np.abs(out - fx["expected"])) < fx["tol"], (out, fx["expected"])


def pin_page_table_example_cache_write(O):
    """Writing each sequence's newest token lands in the hand-derived slot
    and changes nothing else."""
    fx = load_page_table_example()
    kp0, vp0 = fx["kp"].copy(), fx["vp"].copy()
    for (b, r) in fx["slots"]:
        kp0[b, 0, r] = np.nan
        vp0[b, 0, r] = np.nan
    k_new = np.array([[[11.0, 12.0]], [[13.0, 14.0]]], dtype=np.float32)
    v_new = np.array([[[21.0, 22.0]], [[23.0, 24.0]]], dtype=np.float32)
    kp1, vp1 = O.cache_write(kp0, vp0, k_new, v_new, fx["tables"], fx["lens"], fx["bs"])
    exp_k, exp_v = kp0.copy(), vp0.copy()
    for i, (b, r) in enumerate(fx["slots"]):
        exp_k[b, 0, r] = k_new[i, 0]
        exp_v[b, 0, r] = v_new[i, 0]
    assert kp1.tobytes() == exp_k.tobytes()
    assert vp1.tobytes() == exp_v.tobytes()
    assert kp0.tobytes() != kp1.tobytes()        # inputs untouched, outputs changed


def pin_pages_arithmetic(O):
    fx = json.loads((GOLDEN / "pages_arithmetic.json").read_text())
    a = fx["blocks_for_3200_tokens_at_512"]
    assert O.blocks_needed(a["seq_len"], a["block_size"]) == a["expected_blocks"]
    c = fx["pool_capacity_tokens"]
    assert c["num_gpu_blocks"] * c["block_size"] == c["expected_tokens"]
    for L, bs, nb in ((0, 16, 0), (1, 16, 1), (16, 16, 1), (17, 16, 2), (33, 16, 3),
                      (1, 1, 1), (5, 1, 5), (512, 512, 1), (513, 512, 2)):
        assert O.blocks_needed(L, bs) == nb, (L, bs)


# --------------------------------------------------------------- brute force
def _scalar(x, dtype):
    """Decode one stored element to a Python float without numpy casts."""
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<f", float(x)))[0]
    if dtype == "f16":
        return struct.unpack("<e", np.float16(x).tobytes())[0]
    if dtype == "bf16":
        bits = int(x)
        return struct.unpack(">f", bytes([bits >> 8, bits & 0xFF, 0, 0]))[0]
    raise ValueError(dtype)


def brute_force_decode(q, kp, vp, tables, lens, scale, bs, dtype):
    """Scalar paged attention: walk logical token t, find its page through
    the table (page table[t // bs], row t % bs), two-pass softmax with
    math.exp.  No concatenation, no numpy arithmetic."""
    B, Hq, d = q.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    sc = float(np.float32(scale))
    out = np.zeros((B, Hq, d))
    for s in range(B):
        L = int(lens[s])
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            z = []
            for t in range(L):
                blk, row = int(tables[s][t // bs]), t % bs
                acc = 0.0
                for j in range(d):
                    acc += _scalar(q[s, h, j], dtype) * _scalar(kp[blk, g, row, j], dtype)
                z.append(acc * sc)
            m = max(z)
            w = [math.exp(x - m) for x in z]
            tot = math.fsum(w)
            for j in range(d):
                num = math.fsum(w[t] * _scalar(vp[int(tables[s][t // bs]), g, t % bs, j], dtype)
                                for t in range(L))
                out[s, h, j] = num / tot
    return out


def random_tiny_case(rng, B, Lmax, bs, d, Hkv, G, dtype, poison=True):
    """A tiny paged case with a random block placement, built by hand (not
    by the workload generator), plus its logical rows."""
    lens = rng.integers(0, Lmax + 1, size=B)
    nbs = [-(-int(L) // bs) for L in lens]
    NB = sum(nbs) + int(rng.integers(0, 4))
    perm = rng.permutation(NB)
    MB = max(1, max(nbs))
    st = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    nan = {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(0x7FC0)}[dtype]
    kp = np.full((NB, Hkv, bs, d), nan if poison else st(0), dtype=st)
    vp = kp.copy()
    tables = np.full((B, MB), -1, dtype=np.int32)
    q = to_storage(rng.standard_normal((B, Hkv * G, d), dtype=np.float32), dtype)
    lk, lv = [], []
    k = 0
    for s in range(B):
        L = int(lens[s])
        K = to_storage(rng.standard_normal((L, Hkv, d), dtype=np.float32), dtype)
        V = to_storage(rng.standard_normal((L, Hkv, d), dtype=np.float32), dtype)
        for i in range(nbs[s]):
            tables[s, i] = perm[k]
            k += 1
        for t in range(L):
            kp[tables[s, t // bs], :, t % bs, :] = K[t]
            vp[tables[s, t // bs], :, t % bs, :] = V[t]
        lk.append(K)
        lv.append(V)
    scale = np.float32(1.0 / math.sqrt(d))
    return q, kp, vp, tables, lens.astype(np.int32), scale, lk, lv


def pin_brute_force(O, seeds=range(6)):
    for seed in seeds:
        rng = np.random.default_rng(100 + seed)
        for dtype in ("f32", "f16", "bf16"):
            bs = int(rng.choice([1, 2, 4, 16]))
            G = int(rng.choice([1, 2]))
            d = int(rng.integers(1, 9))
            q, kp, vp, tb, lens, scale, _, _ = random_tiny_case(rng, 3, 40, bs, d, 2, G, dtype)
            a = O.decode(q, kp, vp, tb, lens, scale, bs, dtype)
            b = brute_force_decode(q, kp, vp, tb, lens, scale, bs, dtype)
            assert np.all(np.isfinite(a))
            assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b))), (seed, dtype)


# --------------------------------------------------------------- closed forms
def _single_seq(K, V, q, scale=np.float32(0.5)):
    """One sequence, one head, contiguous blocks 0..nb-1, block size 4."""
    L, d = K.shape
    bs = 4
    nb = max(1, -(-L // bs))
    kp = np.full((nb, 1, bs, d), np.nan)
    vp = np.full((nb, 1, bs, d), np.nan)
    for t in range(L):
        kp[t // bs, 0, t % bs] = K[t]
        vp[t // bs, 0, t % bs] = V[t]
    tables = np.arange(nb, dtype=np.int32)[None, :]
    return (np.asarray(q, dtype=np.float64)[None, None, :], kp, vp, tables,
            np.array([L], dtype=np.int32), scale, bs)


def pin_closed_forms(O):
    rng = np.random.default_rng(7)
    d = 5
    # one token: the output is that token's value row, exactly
    K, V, q = rng.standard_normal((1, d)), rng.standard_normal((1, d)), rng.standard_normal(d)
    out = O.decode(*_single_seq(K, V, q), "f32")[0, 0]
    assert np.array_equal(out, V[0])
    # identical keys (or a zero query): uniform weights -> mean of value rows
    K = np.tile(rng.standard_normal(d), (9, 1))
    V = rng.standard_normal((9, d))
    out = O.decode(*_single_seq(K, V, rng.standard_normal(d)), "f32")[0, 0]
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)
    out = O.decode(*_single_seq(rng.standard_normal((9, d)), V, np.zeros(d)), "f32")[0, 0]
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-14)
    # identical value rows: the output is that row, whatever the weights
    c = rng.standard_normal(d)
    out = O.decode(*_single_seq(rng.standard_normal((11, d)) * 3, np.tile(c, (11, 1)),
                                rng.standard_normal(d)), "f32")[0, 0]
    assert np.allclose(out, c, rtol=0, atol=1e-14)
    # two tokens: weight of token 0 is the logistic function of the score gap
    for scale in (np.float32(0.5), np.float32(0.125), np.float32(2.0)):
        K = rng.standard_normal((2, d))
        V = rng.standard_normal((2, d))
        q = rng.standard_normal(d)
        z0, z1 = float(K[0] @ q) * float(scale), float(K[1] @ q) * float(scale)
        w0 = 0.5 * (1.0 + math.tanh((z0 - z1) / 2.0))
        out = O.decode(*_single_seq(K, V, q, scale), "f32")[0, 0]
        assert np.allclose(out, w0 * V[0] + (1 - w0) * V[1], rtol=0, atol=1e-13), scale
    # needle: one score 300 above all others -> that token's value row
    L = 23
    K = np.zeros((L, d))
    K[:, 0] = rng.standard_normal(L)
    needle = 17
    K[needle, 0] = 600.0            # q = e_0, scale 0.5 -> score gap >= ~298
    V = rng.standard_normal((L, d))
    out = O.decode(*_single_seq(K, V, np.eye(d)[0]), "f32")[0, 0]
    assert np.allclose(out, V[needle], rtol=0, atol=1e-100)
    # scores far beyond exp's range in both directions stay finite and exact
    K = np.zeros((3, d))
    K[:, 0] = [4000.0, 3990.0, -5000.0]
    V = rng.standard_normal((3, d))
    out = O.decode(*_single_seq(K, V, np.eye(d)[0], np.float32(1.0)), "f32")[0, 0]
    w = np.array([1.0, math.exp(-10.0), 0.0])
    assert np.allclose(out, (w @ V) / w.sum(), rtol=0, atol=1e-13)
    # empty sequence -> zeros
    out = O.decode(*_single_seq(np.zeros((0, d)), np.zeros((0, d)), np.ones(d)), "f32")
    assert np.array_equal(out, np.zeros((1, 1, d)))


# --------------------------------------------------------------- invariances
def pin_contiguous_equality(O):
    """Paging changes nothing: the paged result equals attention over each
    sequence's contiguous K/V, bit for bit in fp64."""
    for w in (TINY, small_variant(LLAMA7B), small_variant(GQA70B), small_variant(SHARED_PREFIX)):
        c = make_case(w, keep_logical=True)
        a = O.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                     c.block_size, c.dtype)
        b = O.contiguous_attention(c.q, c.logical_k, c.logical_v, c.scale, c.dtype,
                                   w.num_kv_heads)
        assert np.all(np.isfinite(a)), w.name
        assert np.array_equal(a, b), w.name


def relabel_blocks(c, rng):
    """The same logical contents under a different physical placement: block
    b moves to pi[b] and every table entry in use is renamed accordingly."""
    NB = c.k_pool.shape[0]
    pi = rng.permutation(NB)
    kp = np.empty_like(c.k_pool)
    vp = np.empty_like(c.v_pool)
    kp[pi] = c.k_pool
    vp[pi] = c.v_pool
    tb = np.where(c.block_tables >= 0, pi[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    return kp, vp, tb


def pin_permutation_invariance(O):
    rng = np.random.default_rng(11)
    for w in (TINY, small_variant(LONG_BS512), small_variant(GQA70B)):
        c = make_case(w)
        a = O.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                     c.block_size, c.dtype)
        kp, vp, tb = relabel_blocks(c, rng)
        b = O.decode(c.q, kp, vp, tb, c.context_lens, c.scale, c.block_size, c.dtype)
        assert np.array_equal(a, b), w.name


def unshare_prefix(c):
    """Give every sequence private copies of its group's shared prompt
    blocks (appended at the end of the pool) and point its table there."""
    pb = c.prompt_blocks
    B = c.workload.num_seqs
    NB = c.k_pool.shape[0]
    kp = np.concatenate([c.k_pool, np.empty((B * pb,) + c.k_pool.shape[1:], c.k_pool.dtype)])
    vp = np.concatenate([c.v_pool, np.empty((B * pb,) + c.v_pool.shape[1:], c.v_pool.dtype)])
    tb = c.block_tables.copy()
    for s in range(B):
        for i in range(pb):
            new = NB + s * pb + i
            kp[new] = c.k_pool[c.block_tables[s, i]]
            vp[new] = c.v_pool[c.block_tables[s, i]]
            tb[s, i] = new
    return kp, vp, tb


def pin_shared_equals_duplicated(O):
    c = make_case(small_variant(SHARED_PREFIX))
    # the tables really alias: every member of a group lists the same prompt blocks
    for grp in c.shared_groups:
        for s in grp[1:]:
            assert np.array_equal(c.block_tables[s, :c.prompt_blocks],
                                  c.block_tables[grp[0], :c.prompt_blocks])
    a = O.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                 c.block_size, c.dtype)
    kp, vp, tb = unshare_prefix(c)
    assert len(np.unique(tb[tb >= 0])) == int((tb >= 0).sum())   # no aliasing left
    b = O.decode(c.q, kp, vp, tb, c.context_lens, c.scale, c.block_size, c.dtype)
    assert np.array_equal(a, b)


def pin_gqa_equals_repeated_mha(O):
    """Grouped heads equal plain multi-head attention in which every KV head
    is repeated for its G consecutive query heads."""
    c = make_case(small_variant(GQA70B))
    G = c.workload.group_ratio
    a = O.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                 c.block_size, c.dtype)
    kp = np.repeat(c.k_pool, G, axis=1)
    vp = np.repeat(c.v_pool, G, axis=1)
    b = O.decode(c.q, kp, vp, c.block_tables, c.context_lens, c.scale, c.block_size, c.dtype)
    assert np.array_equal(a, b)


def pin_partition_merge(O):
    for w, P in ((small_variant(LONG_BS512), 512), (small_variant(LLAMA7B), 48),
                 (small_variant(GQA70B), 32), (TINY, 16)):
        c = make_case(w)
        a = O.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                     c.block_size, c.dtype)
        b = O.decode_partitioned(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                 c.scale, c.block_size, c.dtype, P)
        assert np.max(np.abs(a - b)) <= 1e-12, w.name


def pin_cache_write_round_trip(O):
    """Writing each sequence's newest token into a pool where that row holds
    NaN restores the fully populated pool byte for byte."""
    for w in (TINY, small_variant(SHARED_PREFIX), small_variant(LONG_BS512)):
        c = make_case(w)
        kp0, vp0 = c.pools_with_new_slots_poisoned()
        assert kp0.tobytes() != c.k_pool.tobytes()
        kp1, vp1 = O.cache_write(kp0, vp0, c.k_new, c.v_new, c.block_tables, c.context_lens,
                                 c.block_size)
        assert kp1.tobytes() == c.k_pool.tobytes(), w.name
        assert vp1.tobytes() == c.v_pool.tobytes(), w.name


def pin_contiguous_cache_write(O):
    """The contiguous layout's write: putting each sequence's newest token
    into a cache whose row L-1 holds NaN gives back the cache the generator
    laid out from its own logical rows, byte for byte; lengths of 0 or past
    the region change nothing."""
    for w in (TINY, small_variant(GQA70B), small_variant(LLAMA7B)):
        c = make_case(w, keep_logical=True)
        max_len = int(c.context_lens.max()) + 3
        kc, vc = contiguous_cache(c, max_len)
        kp0, vp0 = kc.copy(), vc.copy()
        for s, L in enumerate(c.context_lens):
            if L >= 1:
                kp0[s, :, L - 1] = NAN_BITS[w.dtype]
                vp0[s, :, L - 1] = NAN_BITS[w.dtype]
        assert kp0.tobytes() != kc.tobytes()
        k1, v1 = O.cache_write_contiguous(kp0, vp0, c.k_new, c.v_new, c.context_lens)
        assert k1.tobytes() == kc.tobytes() and v1.tobytes() == vc.tobytes(), w.name
        # lengths that write nothing
        lens = c.context_lens.copy()
        lens[:] = 0
        lens[-1] = max_len + 1
        k2, v2 = O.cache_write_contiguous(kp0, vp0, c.k_new, c.v_new, lens)
        assert k2.tobytes() == kp0.tobytes() and v2.tobytes() == vp0.tobytes(), w.name


ALL_PINS = [pin_page_table_example, pin_page_table_example_cache_write, pin_pages_arithmetic,
            pin_brute_force, pin_closed_forms, pin_contiguous_equality,
            pin_permutation_invariance, pin_shared_equals_duplicated,
            pin_gqa_equals_repeated_mha, pin_partition_merge, pin_cache_write_round_trip,
            pin_contiguous_cache_write]
