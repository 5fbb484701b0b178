"""Synthetic paged-decode workloads.

Each workload fixes the shapes, dtype, length mix and pool layout of one
decode step of one attention layer.  The pages measure on no public dataset,
so every input here is drawn from a seeded generator (see ``gen.py``).

Shapes follow the paging structure of the pages: a pool of fixed-size blocks
("IO-5 vLLM Paged Attention", section 3 "KV Cache Paging structure") and one
block table per sequence (same page, section 2 "Paged Attention idea").  The
large-page workload uses the page size the deployment tips recommend ("vLLM's
efficiency secret: PagedAttention and dynamic memory management", section
"Deployment tips").

This module holds no attention arithmetic; it only describes workloads.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_heads: int            # query heads
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                # "f32" | "f16" | "bf16"
    seed: int
    # length distribution
    length_kind: str          # "fixed" | "uniform" | "lognormal" | "shared_prefix"
    lengths: Tuple[int, ...] = ()          # for "fixed"
    length_lo: int = 0                      # uniform / clip low / suffix low
    length_hi: int = 0                      # uniform / clip high / suffix high
    lognormal_median: float = 0.0
    lognormal_sigma: float = 0.0
    # shared prefix (parallel sampling): groups x group_size sequences
    groups: int = 0
    group_size: int = 0
    prompt_len: int = 0
    # value distributions (standard deviations)
    q_std: float = 1.0
    kv_std: float = 1.0
    # pool
    num_blocks: Optional[int] = None        # fixed pool size, else pool_factor x used blocks
    pool_factor: int = 2
    max_blocks_per_seq: int = 0
    # split-K partition size used by the workload (None: single pass)
    partition_size: Optional[int] = None
    cache_write: bool = True
    description: str = ""

    @property
    def group_ratio(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = Workload(
    name="tiny", num_seqs=4, num_heads=2, num_kv_heads=2, head_dim=64,
    block_size=16, dtype="f32", seed=0, length_kind="fixed",
    lengths=(1, 7, 16, 33), num_blocks=16, max_blocks_per_seq=3,
    description="4 seqs, L={1,7,16,33}, 2 heads, d=64, bs=16, f32, pool of 16 blocks",
)

LLAMA7B = Workload(
    name="llama2_7b", num_seqs=64, num_heads=32, num_kv_heads=32, head_dim=128,
    block_size=16, dtype="f16", seed=1, length_kind="uniform",
    length_lo=128, length_hi=2048, max_blocks_per_seq=128,
    description="Llama-2-7B-shaped layer: B=64, 32 heads MHA, d=128, bs=16, fp16, "
                "L~U[128,2048], 2x shuffled pool",
)

LONG_BS512 = Workload(
    name="long_bs512", num_seqs=16, num_heads=32, num_kv_heads=32, head_dim=128,
    block_size=512, dtype="bf16", seed=2, length_kind="uniform",
    length_lo=8192, length_hi=32768, max_blocks_per_seq=64, partition_size=512,
    description="long context, 512-token pages: B=16, 32 heads, d=128, bf16, "
                "L~U[8192,32768], split-K P=512",
)

GQA70B = Workload(
    name="gqa_70b", num_seqs=256, num_heads=64, num_kv_heads=8, head_dim=128,
    block_size=16, dtype="bf16", seed=3, length_kind="lognormal",
    lognormal_median=1024.0, lognormal_sigma=1.0, length_lo=16, length_hi=16384,
    kv_std=0.5 ** 0.5, max_blocks_per_seq=1024,
    description="GQA 70B-shaped layer: B=256, 64 q heads / 8 kv heads, d=128, bs=16, "
                "bf16, L log-normal (median 1024, sigma 1) clipped to [16,16384], "
                "K/V ~ N(0, variance 0.5)",
)

SHARED_PREFIX = Workload(
    name="shared_prefix", num_seqs=256, num_heads=32, num_kv_heads=32, head_dim=128,
    block_size=16, dtype="f16", seed=4, length_kind="shared_prefix",
    groups=32, group_size=8, prompt_len=1024, length_lo=64, length_hi=256,
    max_blocks_per_seq=80,
    description="parallel sampling: 32 groups x 8 seqs sharing a 1024-token prompt's "
                "blocks, suffixes U[64,256] tokens, 32 heads, d=128, bs=16, fp16",
)

WORKLOADS = {w.name: w for w in (TINY, LLAMA7B, LONG_BS512, GQA70B, SHARED_PREFIX)}


def small_variant(w: Workload) -> Workload:
    """A scaled-down workload with the same structure (dtype, head grouping,
    block size, length mix shape) that the fp64 oracle finishes in seconds,
    while still spanning several blocks and partitions and a ragged tail."""
    if w.name == "tiny":
        return w
    if w.name == "llama2_7b":
        return w.replace(name="llama2_7b_small", num_seqs=6, num_heads=4, num_kv_heads=4,
                         length_lo=1, length_hi=300, max_blocks_per_seq=19)
    if w.name == "long_bs512":
        return w.replace(name="long_bs512_small", num_seqs=3, num_heads=2, num_kv_heads=2,
                         length_lo=700, length_hi=2600, max_blocks_per_seq=6)
    if w.name == "gqa_70b":
        return w.replace(name="gqa_70b_small", num_seqs=6, num_heads=16, num_kv_heads=2,
                         lognormal_median=100.0, length_lo=1, length_hi=400,
                         max_blocks_per_seq=25)
    if w.name == "shared_prefix":
        return w.replace(name="shared_prefix_small", num_seqs=6, num_heads=4, num_kv_heads=4,
                         groups=2, group_size=3, prompt_len=64, length_lo=5, length_hi=40,
                         max_blocks_per_seq=7)
    raise KeyError(w.name)
