"""CPU tests of the seeded workload generator (structure and determinism)."""
import numpy as np
import pytest
import torch

from synthetic import (GQA70B, LLAMA7B, LONG_BS512, SHARED_PREFIX, TINY, WORKLOADS,
                       algorithmic_bytes, ceil_div, contiguous_cache, f32_to_bf16_bits, make_case,
                       small_variant)

SMALL = [small_variant(w) for w in WORKLOADS.values()]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_determinism(w):
    a, b = make_case(w), make_case(w)
    assert a.digest() == b.digest()
    assert make_case(w, seed=w.seed + 1000).digest() != a.digest()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_structure(w):
    c = make_case(w, keep_logical=True)
    B, bs = w.num_seqs, w.block_size
    lens = c.context_lens
    assert lens.dtype == np.int32 and c.block_tables.dtype == np.int32
    used = []
    for s in range(B):
        nb = ceil_div(int(lens[s]), bs)
        row = c.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < c.num_blocks)
        assert np.all(row[nb:] == -1)
        used.extend(row[:nb].tolist())
        # logical rows sit where the table says
        for t in range(0, int(lens[s]), max(1, int(lens[s]) // 7)):
            blk, r = row[t // bs], t % bs
            assert c.k_pool[blk, :, r].tobytes() == c.logical_k[s][t].tobytes()
            assert c.v_pool[blk, :, r].tobytes() == c.logical_v[s][t].tobytes()
        if lens[s] > 0:
            assert c.k_new[s].tobytes() == c.logical_k[s][-1].tobytes()
            assert tuple(c.new_slots[s]) == (row[(lens[s] - 1) // bs], (lens[s] - 1) % bs)
    uniq = set(used)
    assert len(uniq) == c.unique_blocks
    if w.length_kind != "shared_prefix":
        assert len(used) == len(uniq)              # no aliasing
    else:
        assert len(used) == len(uniq) + (w.group_size - 1) * w.groups * c.prompt_blocks
    if w.num_blocks is None:
        assert c.num_blocks == 2 * c.unique_blocks
    # unused blocks and tail rows are poisoned
    free = sorted(set(range(c.num_blocks)) - uniq)
    if free:
        kb = c.k_pool[free]
        if w.dtype == "bf16":
            assert np.all(kb == 0x7FC0)
        else:
            assert np.all(np.isnan(kb))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_contiguous_cache_layout(w):
    """Row t of KV head g in sequence s's region is the same bytes as the pool
    row the table names for it; rows past the length are NaN."""
    c = make_case(w, keep_logical=True)
    extra = 5
    max_len = int(c.context_lens.max()) + extra
    kc, vc = contiguous_cache(c, max_len)
    assert kc.shape == (w.num_seqs, w.num_kv_heads, max_len, w.head_dim) == vc.shape
    assert kc.dtype == c.k_pool.dtype
    bs = w.block_size
    for s in range(w.num_seqs):
        L = int(c.context_lens[s])
        for t in range(L):
            blk, r = c.block_tables[s, t // bs], t % bs
            assert kc[s, :, t].tobytes() == c.k_pool[blk, :, r].tobytes()
            assert vc[s, :, t].tobytes() == c.v_pool[blk, :, r].tobytes()
        tail = kc[s, :, L:]
        assert np.all(tail == 0x7FC0) if w.dtype == "bf16" else np.all(np.isnan(tail))
    with pytest.raises(ValueError):
        contiguous_cache(c, int(c.context_lens.max()) - 1)
    with pytest.raises(ValueError):
        contiguous_cache(make_case(w), max_len)          # logical rows not kept


def test_contiguous_cache_on_a_torch_device_matches_host():
    """The device builder (here on the CPU device) lays out the same bits."""
    for w in (small_variant(GQA70B), small_variant(LLAMA7B)):
        c = make_case(w, keep_logical=True)
        kc, vc = contiguous_cache(c, int(c.context_lens.max()) + 3)
        kt, vt = contiguous_cache(c, int(c.context_lens.max()) + 3, device="cpu")
        for host, dev in ((kc, kt), (vc, vt)):
            bits = dev.view(torch.int16).numpy() if dev.dtype == torch.bfloat16 else dev.numpy()
            assert bits.tobytes() == host.tobytes()


def test_lengths_follow_workloads():
    c = make_case(TINY)
    assert c.context_lens.tolist() == [1, 7, 16, 33]
    assert c.num_blocks == 16
    rng = np.random.default_rng(LLAMA7B.seed)
    from synthetic.gen import draw_lengths
    L = draw_lengths(LLAMA7B, rng)
    assert L.min() >= 128 and L.max() <= 2048 and len(L) == 64
    L = draw_lengths(GQA70B, np.random.default_rng(GQA70B.seed))
    assert L.min() >= 16 and L.max() <= 16384 and 500 < np.median(L) < 2000
    L = draw_lengths(LONG_BS512, np.random.default_rng(LONG_BS512.seed))
    assert L.min() >= 8192 and L.max() <= 32768
    L = draw_lengths(SHARED_PREFIX, np.random.default_rng(SHARED_PREFIX.seed))
    assert L.min() >= 1024 + 64 and L.max() <= 1024 + 256


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 100
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_algorithmic_bytes_tiny():
    c = make_case(TINY)
    # 57 tokens x 2 (K,V) x 2 heads x 64 x 4 B + Q,out 2x4x2x64x4 + 4*(6 blocks + 4 lens)
    assert algorithmic_bytes(c) == 57 * 2 * 2 * 64 * 4 + 2 * 4 * 2 * 64 * 4 + 4 * (6 + 4)


def test_shared_prefix_unique_bytes():
    w = small_variant(SHARED_PREFIX)
    c = make_case(w)
    logical = algorithmic_bytes(c)
    unique = algorithmic_bytes(c, unique=True)
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    assert logical - unique == (w.group_size - 1) * w.groups * w.prompt_len * per_tok
