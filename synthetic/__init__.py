"""Seeded synthetic workloads for paged decode attention (no attention arithmetic)."""
from .configs import Workload, WORKLOADS, TINY, LLAMA7B, LONG_BS512, GQA70B, SHARED_PREFIX, small_variant
from .gen import (Case, make_case, to_storage, f32_to_bf16_bits, ceil_div, kv_token_count,
                  algorithmic_bytes, contiguous_cache, STORAGE, NAN_BITS)
