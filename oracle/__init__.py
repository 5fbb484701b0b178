"""fp64 CPU oracle for paged decode attention.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg import this package.  It shares no code with the HIP path.
"""
from .paged_attention import (widen, blocks_needed, gather_kv, softmax_attention, decode,
                              decode_partitioned, cache_write, cache_write_contiguous,
                              contiguous_attention)
from .block_ops import copy_blocks, swap_blocks
