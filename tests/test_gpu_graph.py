"""A whole decode step captured in a HIP graph (torch.cuda.CUDAGraph over
the library's calls on the capture stream) and replayed, as a serving loop
would run it.  The combined entries launch kernels only -- no allocation,
no memset, no copy -- so the captured step is those launches.

Each replay is checked against the eager call: pools byte for byte, output
bit for bit.  Replays alternate with eager work and synchronisations, and
the inputs change between replays (the query heads are permuted and the new
rows rolled; lengths are part of the capture's arguments only through the
device array, which stays), so a replay that reused stale results would be
caught.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_438_amd as pa
from synthetic import GQA70B, LLAMA7B, SHARED_PREFIX, make_case, small_variant
from tests.gpu_util import DevCase, dev_array, host_bits, note

pytestmark = pytest.mark.gpu


def _groups(c):
    seq_group = np.full(c.workload.num_seqs, -1, dtype=np.int32)
    for gi, members in enumerate(c.shared_groups):
        seq_group[members] = gi
    prefix = np.full(len(c.shared_groups), c.workload.prompt_len, dtype=np.int32)
    return dev_array(seq_group), dev_array(prefix), int(c.shared_groups.shape[1])


def _step_fn(d, kind, out, ws):
    c = d.c
    sc = float(c.scale)
    maxlen = int(c.context_lens.max())
    if kind == "single":
        return lambda: pa.pa_write_decode(d.q, d.k_pool, d.v_pool, d.k_new, d.v_new, d.tables,
                                          d.lens, scale=sc, out=out)
    if kind == "splitk":
        return lambda: pa.pa_write_decode_splitk(d.q, d.k_pool, d.v_pool, d.k_new, d.v_new,
                                                 d.tables, d.lens, partition_size=64,
                                                 max_context_len=maxlen, scale=sc, out=out,
                                                 workspace=ws)
    sg, pl, mg = _groups(c)
    return lambda: pa.pa_write_decode_shared_prefix(d.q, d.k_pool, d.v_pool, d.k_new, d.v_new,
                                                    d.tables, d.lens, sg, pl, mg, 64, maxlen,
                                                    scale=sc, out=out, workspace=ws)


@pytest.mark.parametrize("w,kind", [(small_variant(LLAMA7B), "single"),
                                    (small_variant(GQA70B), "splitk"),
                                    (small_variant(SHARED_PREFIX), "shared")],
                         ids=["llama2_7b_single", "gqa_70b_splitk", "shared_prefix"])
def test_captured_step_replays_like_eager(w, kind):
    c = make_case(w)
    kp0, vp0 = c.pools_with_new_slots_poisoned()
    g_case = DevCase(c, k_pool=kp0, v_pool=vp0)        # the graph's buffers
    e_case = DevCase(c, k_pool=kp0, v_pool=vp0)        # eager reference
    maxlen = int(c.context_lens.max())
    if kind == "single":
        need = 0
    elif kind == "splitk":
        need = pa.pa_decode_splitk_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim, maxlen,
                                                   64)
    else:
        need = pa.pa_decode_shared_prefix_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim,
                                                          maxlen, 64, len(c.shared_groups))
    g_ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    e_ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    g_out = torch.empty_like(g_case.q)
    e_out = torch.empty_like(e_case.q)
    g_step = _step_fn(g_case, kind, g_out, g_ws)
    e_step = _step_fn(e_case, kind, e_out, e_ws)

    # Warm up on a side stream (library and kernel loading), then capture.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        g_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(17)
    for rep in range(4):
        note(f"graph replay {rep}: {w.name} {kind}")
        if rep > 0:
            # the same new inputs for both copies: query heads permuted and
            # the new rows rolled across sequences
            perm = torch.from_numpy(rng.permutation(w.num_heads)).cuda()
            for d in (g_case, e_case):
                d.q.copy_(d.q[:, perm].contiguous())
                d.k_new.copy_(d.k_new.roll(1, dims=0).contiguous())
                d.v_new.copy_(d.v_new.roll(1, dims=0).contiguous())
        graph.replay()
        e_step()
        torch.cuda.synchronize()
        assert host_bits(g_out).tobytes() == host_bits(e_out).tobytes(), f"replay {rep}: output"
        assert host_bits(g_case.k_pool).tobytes() == host_bits(e_case.k_pool).tobytes()
        assert host_bits(g_case.v_pool).tobytes() == host_bits(e_case.v_pool).tobytes()
        # the program's own eager work between replays
        _ = (g_out.float().sum() + e_out.float().sum()).item()
