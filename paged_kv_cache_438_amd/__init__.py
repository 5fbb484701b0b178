"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The computation runs in libpa.so (hand-written HIP kernels behind the C ABI
in include/pa.h); this package is its thin Python binding.
"""
from .block_manager import BlockManager, OutOfBlocks
from ._binding import (PA_BF16, PA_F16, PA_F32, PA_FLAG_SHARED_KV, PA_FLAG_VALU_ONLY, PA_NOALLOC_SCRATCH_BYTES, PaError, abi_version, header_functions,
                       last_error, load, pa_cache_write, pa_check_inputs_host, pa_decode,
                       pa_decode_shared_prefix, pa_decode_shared_prefix_workspace_bytes,
                       pa_decode_contiguous, pa_cache_write_contiguous, pa_copy_blocks, pa_device_memory, pa_read_probe, pa_swap_blocks,
                       pa_decode_splitk, pa_decode_splitk_noalloc, pa_decode_splitk_workspace_bytes,
                       pa_write_decode, pa_write_decode_splitk, pa_write_decode_shared_prefix,
                       status_str, LIB_PATH)

__all__ = ["pa_cache_write", "pa_decode", "pa_decode_splitk", "pa_decode_splitk_noalloc",
           "pa_decode_splitk_workspace_bytes", "PA_NOALLOC_SCRATCH_BYTES",
           "pa_decode_shared_prefix", "pa_decode_shared_prefix_workspace_bytes",
           "pa_decode_contiguous", "pa_cache_write_contiguous", "pa_write_decode", "pa_write_decode_splitk",
           "pa_write_decode_shared_prefix", "pa_check_inputs_host", "PaError", "load", "abi_version", "status_str", "last_error",
           "header_functions", "PA_F32", "PA_F16", "PA_BF16", "PA_FLAG_SHARED_KV", "PA_FLAG_VALU_ONLY",
           "LIB_PATH", "BlockManager", "OutOfBlocks", "pa_copy_blocks", "pa_swap_blocks",
           "pa_read_probe", "pa_device_memory"]
