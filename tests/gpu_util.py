"""Helpers for the GPU parity tests: move seeded host cases to the device and
read results back as fp64.  No attention arithmetic here."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_438_amd as pa

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# Max-abs error bounds against the fp64 oracle, fp32 accumulation.
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}


def note(msg: str) -> None:
    print(msg, flush=True)


def dev_array(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a device tensor as a host array (uint16 bits for bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        b = t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    return t.numpy().astype(np.float64)


class DevCase:
    """Device copies of a synthetic case."""

    def __init__(self, c, k_pool=None, v_pool=None, tables=None):
        self.c = c
        dt = c.dtype
        self.q = dev_array(c.q, dt)
        self.k_pool = dev_array(c.k_pool if k_pool is None else k_pool, dt)
        self.v_pool = dev_array(c.v_pool if v_pool is None else v_pool, dt)
        self.tables = dev_array(c.block_tables if tables is None else tables)
        self.lens = dev_array(c.context_lens)
        self.k_new = dev_array(c.k_new, dt)
        self.v_new = dev_array(c.v_new, dt)

    def decode(self, entry: str, partition_size: int = None, scale=None, shared_kv=False,
               valu_only=False):
        sc = float(self.c.scale) if scale is None else scale
        if entry == "single":
            return pa.pa_decode(self.q, self.k_pool, self.v_pool, self.tables, self.lens, scale=sc,
                                shared_kv=shared_kv, valu_only=valu_only)
        P = partition_size or 256
        return pa.pa_decode_splitk(self.q, self.k_pool, self.v_pool, self.tables, self.lens,
                                   partition_size=P,
                                   max_context_len=int(self.c.context_lens.max(initial=0)),
                                   scale=sc, shared_kv=shared_kv, valu_only=valu_only)

    def cache_write(self):
        pa.pa_cache_write(self.k_pool, self.v_pool, self.k_new, self.v_new, self.tables, self.lens)
