"""Seeded random sweep of decode configurations on the GPU against the fp64
oracle.

Each case draws its own shape from a counter-seeded generator: dtype,
head_dim, KV heads, query heads per KV head (1 to 16, including ones that do
not divide 16), block size 1 to 256, batch, a length mix with zeros and block
boundaries, and the entry point (single pass, split-K at one of seven
partition sizes, the vector-ALU-only flag, sharing-aware decode over random
prompt groups, decode over a contiguous cache with a random region length,
or a whole step -- the new token's write and the decode in one call).  The
case is printed before it runs, so a failure names its draw.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_438_amd as pa
from synthetic import SHARED_PREFIX, TINY, contiguous_cache, make_case
from tests.gpu_util import TOL, DevCase, dev_array, host_bits, host_f64, note

pytestmark = pytest.mark.gpu

N_PLAIN = 60
N_SHARED = 24
N_CONTIGUOUS = 24
N_STEP = 24


def _plain_case(i):
    rng = np.random.default_rng(70_000 + i)
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256]))
    B = int(rng.integers(1, 10))
    cap = int(rng.choice([20, 100, 400, 900]))
    lens = rng.integers(0, cap + 1, size=B)
    specials = [0, 1, bs, bs + 1, max(bs - 1, 1), cap]
    for j in range(B):
        if rng.random() < 0.3:
            lens[j] = min(int(rng.choice(specials)), cap)
    mb = max(1, -(-int(lens.max()) // bs)) + int(rng.integers(0, 3))
    used = int(sum(-(-int(L) // bs) for L in lens))
    entry = str(rng.choice(["single", "splitk", "single_valu", "splitk_valu"]))
    P = int(rng.choice([16, 32, 48, 64, 128, 256, 512]))
    w = TINY.replace(name=f"sweep{i}", num_seqs=B, num_heads=hkv * G, num_kv_heads=hkv,
                     head_dim=d, block_size=bs, dtype=dtype, seed=80_000 + i,
                     length_kind="fixed", lengths=tuple(int(x) for x in lens),
                     num_blocks=2 * used + 3, max_blocks_per_seq=mb)
    return w, entry, P


def _shared_case(i):
    rng = np.random.default_rng(90_000 + i)
    dtype = str(rng.choice(["f16", "bf16"]))
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    bs = int(rng.choice([1, 4, 16, 32, 64]))
    groups = int(rng.integers(1, 4))
    gsize = int(rng.integers(1, 9))
    prompt = bs * int(rng.integers(1, max(2, 200 // bs)))
    lo = int(rng.integers(1, 40))
    hi = lo + int(rng.integers(0, 200))
    P = int(rng.choice([16, 48, 64, 256, 512, 2048]))
    mb = -(-(prompt + hi) // bs) + int(rng.integers(0, 2))
    w = SHARED_PREFIX.replace(name=f"sweep_shared{i}", num_seqs=groups * gsize,
                              num_heads=hkv * G, num_kv_heads=hkv, head_dim=d, block_size=bs,
                              dtype=dtype, seed=95_000 + i, groups=groups, group_size=gsize,
                              prompt_len=prompt, length_lo=lo, length_hi=hi,
                              max_blocks_per_seq=mb)
    return w, P


def _check(got, ref, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    note(f"  {what}: max|err| = {err:.3e} (bound {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], f"{what}: max abs error {err} > {TOL[dtype]}"


@pytest.mark.parametrize("i", range(N_PLAIN))
def test_random_decode_matches_oracle(i):
    w, entry, P = _plain_case(i)
    c = make_case(w)
    note(f"sweep {i}: {w.dtype} d={w.head_dim} Hq={w.num_heads} Hkv={w.num_kv_heads} "
         f"bs={w.block_size} lens={list(w.lengths)} MB={w.max_blocks_per_seq} "
         f"entry={entry} P={P}")
    d = DevCase(c)
    valu = entry.endswith("_valu")
    got = host_f64(d.decode(entry.split("_")[0], partition_size=P, valu_only=valu))
    torch.cuda.synchronize()
    ref = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                        c.block_size, c.dtype)
    _check(got, ref, w.dtype, f"sweep {i}")


@pytest.mark.parametrize("i", range(N_SHARED))
def test_random_shared_prefix_matches_oracle(i):
    w, P = _shared_case(i)
    c = make_case(w)
    B = w.num_seqs
    seq_group = np.full(B, -1, dtype=np.int32)
    for gi, members in enumerate(c.shared_groups):
        seq_group[members] = gi
    prefix = np.full(len(c.shared_groups), w.prompt_len, dtype=np.int32)
    mg = int(c.shared_groups.shape[1])
    note(f"sweep shared {i}: {w.dtype} d={w.head_dim} Hq={w.num_heads} Hkv={w.num_kv_heads} "
         f"bs={w.block_size} groups={w.groups}x{w.group_size} prompt={w.prompt_len} "
         f"lens={c.context_lens.tolist()} P={P}")
    d = DevCase(c)
    got = host_f64(pa.pa_decode_shared_prefix(d.q, d.k_pool, d.v_pool, d.tables, d.lens,
                                              dev_array(seq_group), dev_array(prefix), mg, P,
                                              int(c.context_lens.max()), scale=float(c.scale)))
    torch.cuda.synchronize()
    ref = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                        c.block_size, c.dtype)
    _check(got, ref, w.dtype, f"sweep shared {i}")


@pytest.mark.parametrize("i", range(N_CONTIGUOUS))
def test_random_contiguous_matches_oracle_and_paged(i):
    """pa_decode_contiguous on a random shape, with a region 0 to 40 rows
    longer than the longest sequence: within the bound of the oracle's
    attention over the logical rows, and bit-identical to the paged entry on
    the same rows."""
    w, entry, P = _plain_case(1000 + i)
    c = make_case(w, keep_logical=True)
    extra = int(np.random.default_rng(99_000 + i).integers(0, 41))
    max_len = max(1, int(c.context_lens.max()) + extra)
    part = 0 if entry.startswith("single") else P
    valu = entry.endswith("_valu")
    note(f"sweep contiguous {i}: {w.dtype} d={w.head_dim} Hq={w.num_heads} "
         f"Hkv={w.num_kv_heads} lens={list(w.lengths)} max_len={max_len} P={part} valu={valu}")
    d = DevCase(c)
    kc, vc = contiguous_cache(c, max_len, device="cuda")
    got = pa.pa_decode_contiguous(d.q, kc, vc, d.lens, scale=float(c.scale), partition_size=part,
                                  valu_only=valu)
    paged = d.decode("single" if part == 0 else "splitk", partition_size=part or None,
                     valu_only=valu)
    torch.cuda.synchronize()
    ref = oracle.contiguous_attention(c.q, c.logical_k, c.logical_v, c.scale, c.dtype,
                                      w.num_kv_heads)
    _check(host_f64(got), ref, w.dtype, f"sweep contiguous {i}")
    assert host_bits(got).tobytes() == host_bits(paged).tobytes(), f"sweep contiguous {i}"


@pytest.mark.parametrize("i", range(N_STEP))
def test_random_write_decode_step(i):
    """A whole step in one call (pa_write_decode, pa_write_decode_splitk or
    pa_write_decode_shared_prefix) from pools whose new-token slots hold NaN:
    the pools byte for byte against the oracle's write, the output within the
    bound of the oracle and bit for bit equal to pa_cache_write followed by
    the decode call."""
    shared = i % 2 == 1
    if shared:
        w, P = _shared_case(2000 + i)
        entry = "shared"
    else:
        w, entry, P = _plain_case(2000 + i)
        if i % 4 == 0:
            # one query head per KV head on blocks of 16 tokens or more: the
            # single pass then writes inside the decode launch
            bs = max(16, w.block_size)
            used = sum(-(-L // bs) for L in w.lengths)
            w = w.replace(num_heads=w.num_kv_heads, block_size=bs, num_blocks=2 * used + 3,
                          max_blocks_per_seq=max(1, -(-max(w.lengths) // bs)) + 1)
            entry = "single" if i % 8 == 0 else entry
    c = make_case(w)
    valu = entry.endswith("_valu")
    kind = entry.split("_")[0]
    maxlen = int(c.context_lens.max(initial=0))
    note(f"sweep step {i}: {w.dtype} d={w.head_dim} Hq={w.num_heads} Hkv={w.num_kv_heads} "
         f"bs={w.block_size} lens={c.context_lens.tolist()} entry={entry} P={P}")
    kp0, vp0 = c.pools_with_new_slots_poisoned()
    a = DevCase(c, k_pool=kp0, v_pool=vp0)
    b = DevCase(c, k_pool=kp0, v_pool=vp0)
    sc = float(c.scale)
    if kind == "shared":
        seq_group = np.full(w.num_seqs, -1, dtype=np.int32)
        for gi, members in enumerate(c.shared_groups):
            seq_group[members] = gi
        sg = dev_array(seq_group)
        pl = dev_array(np.full(len(c.shared_groups), w.prompt_len, dtype=np.int32))
        mg = int(c.shared_groups.shape[1])
        got = pa.pa_write_decode_shared_prefix(a.q, a.k_pool, a.v_pool, a.k_new, a.v_new,
                                               a.tables, a.lens, sg, pl, mg, P, maxlen, scale=sc)
        pa.pa_cache_write(b.k_pool, b.v_pool, b.k_new, b.v_new, b.tables, b.lens)
        sep = pa.pa_decode_shared_prefix(b.q, b.k_pool, b.v_pool, b.tables, b.lens, sg, pl, mg,
                                         P, maxlen, scale=sc)
    elif kind == "single":
        got = pa.pa_write_decode(a.q, a.k_pool, a.v_pool, a.k_new, a.v_new, a.tables, a.lens,
                                 scale=sc, valu_only=valu)
        pa.pa_cache_write(b.k_pool, b.v_pool, b.k_new, b.v_new, b.tables, b.lens)
        sep = pa.pa_decode(b.q, b.k_pool, b.v_pool, b.tables, b.lens, scale=sc, valu_only=valu)
    else:
        got = pa.pa_write_decode_splitk(a.q, a.k_pool, a.v_pool, a.k_new, a.v_new, a.tables,
                                        a.lens, partition_size=P, max_context_len=maxlen,
                                        scale=sc, valu_only=valu)
        pa.pa_cache_write(b.k_pool, b.v_pool, b.k_new, b.v_new, b.tables, b.lens)
        sep = pa.pa_decode_splitk(b.q, b.k_pool, b.v_pool, b.tables, b.lens, partition_size=P,
                                  max_context_len=maxlen, scale=sc, valu_only=valu)
    torch.cuda.synchronize()
    ek, ev = oracle.cache_write(kp0, vp0, c.k_new, c.v_new, c.block_tables, c.context_lens,
                                c.block_size)
    assert host_bits(a.k_pool).tobytes() == ek.tobytes(), f"sweep step {i}: K pool"
    assert host_bits(a.v_pool).tobytes() == ev.tobytes(), f"sweep step {i}: V pool"
    ref = oracle.decode(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                        c.block_size, c.dtype)
    _check(host_f64(got), ref, w.dtype, f"sweep step {i}")
    assert host_bits(got).tobytes() == host_bits(sep).tobytes(), f"sweep step {i}: bits"
