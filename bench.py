"""Benchmark: one paged decode step = new-token cache write + decode attention
over a synthetic batch resident in HBM, on one MI355X.

Prints ONE JSON line (last line of stdout).  ``value`` is the step's
algorithmic bytes (K/V rows actually attended, Q, output, table entries,
lengths, plus the cache write's reads and writes) per second of wall time
over the timed steps.  ``roofline`` reports the timed call: the decode, or
for split-K and shared-prompt workloads the one call that writes and
decodes; its algorithmic bytes are divided by its average duration from HIP
events recorded on the stream it runs on.  No event sits between the timed
steps: the events bracket the K timed steps (one call per step), or K more
decode launches run back to back after them (write and decode as two
calls).  ``cpu_baseline`` is the fp64 oracle on host cores over the same
workload, measured before the GPU is touched.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import pathlib
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from synthetic import (WORKLOADS, algorithmic_bytes, contiguous_cache, kv_token_count,  # noqa: E402
                       make_case)

HBM_PEAK_GBS = 8000.0
# Max-abs error bounds against the fp64 oracle, fp32 accumulation.
TOLERANCE = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
METRIC = "paged decode attention: achieved HBM GB/s (% of peak) and KV tokens/sec"
# Entry point and partition size per workload.  The long-context workload is
# specified with 512-token partitions; the grouped-query batch uses 8192-token
# partitions, the best trade between balance and per-partition overhead for
# its log-normal length mix (lengths up to 16384); sharing-aware decode cuts
# each group's 1024-token prompt plus absorbed suffixes into 2048-token units.
DEFAULT_ENTRY = {"llama2_7b": ("single", None), "long_bs512": ("splitk", 512),
                 "gqa_70b": ("splitk", 8192), "shared_prefix": ("shared", 2048),
                 "tiny": ("single", None)}
ENTRY_NAME = {"single": "pa_decode", "splitk": "pa_decode_splitk",
              "shared": "pa_decode_shared_prefix", "contiguous": "pa_decode_contiguous",
              "single_combined": "pa_write_decode",
              "splitk_combined": "pa_write_decode_splitk",
              "shared_combined": "pa_write_decode_shared_prefix"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- CPU baseline
_CASE = None


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _oracle_one(s):
    import oracle
    c = _CASE
    o = oracle.decode(c.q[s:s + 1], c.k_pool, c.v_pool, c.block_tables[s:s + 1],
                      c.context_lens[s:s + 1], c.scale, c.block_size, c.dtype)
    return s, o


def _assemble(case, res) -> np.ndarray:
    """Oracle rows from a pool pass, as one fp64 [B][Hq][d] array."""
    w = case.workload
    ref = np.full((w.num_seqs, w.num_heads, w.head_dim), np.nan, dtype=np.float64)
    for s, o in res:
        ref[s] = o[0]
    return ref


def _workers() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(avail, 16))


def oracle_reference(case) -> np.ndarray:
    """One fp64 oracle pass over every (sequence, head) row, for the check
    of the timed output when the CPU baseline is not measured."""
    global _CASE
    _CASE = case
    order = list(np.argsort(-case.context_lens.astype(np.int64)))
    with mp.get_context("fork").Pool(_workers(), initializer=_worker_init) as pool:
        return _assemble(case, pool.map(_oracle_one, order, chunksize=1))


def cpu_baseline(case, min_seconds: float):
    """Time the fp64 oracle over whole passes of the workload (all sequences,
    all heads) with a fork pool, until at least ``min_seconds`` have passed.
    Returns the last pass's output (every row) and the baseline record."""
    global _CASE
    _CASE = case
    workers = _workers()
    B = case.workload.num_seqs
    tokens = kv_token_count(case)
    order = list(np.argsort(-case.context_lens.astype(np.int64)))   # longest first
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_worker_init) as pool:
        passes = 0
        t0 = time.perf_counter()
        while True:
            res = pool.map(_oracle_one, order, chunksize=1)
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= 1000:
                break
    assert len(res) == B
    ref = _assemble(case, res)
    # The same passes in this process alone, BLAS held to one thread: the
    # single-core rate.
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None
    t1 = time.perf_counter()
    passes1 = 0
    while True:
        for s in order:
            _oracle_one(s)
        passes1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= min(3.0, min_seconds) or passes1 >= 1000:
            break
    if limit is not None:
        limit.restore_original_limits()
    cpu_model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu_model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return ref, {
        "value": passes * tokens / el, "unit": "KV tokens/s", "cores": workers, "kind": "oracle",
        "sample": f"{passes} full pass(es) over all {B} sequences x "
                  f"{case.workload.num_heads} heads ({tokens} KV tokens per pass), "
                  f"fp64 NumPy, fork pool of {workers} workers, {el:.1f} s wall",
        "cpu_model": cpu_model, "os_cpu_count": os.cpu_count(),
        "one_worker": {"value": passes1 * tokens / el1, "unit": "KV tokens/s", "cores": 1,
                       "sample": f"{passes1} full pass(es) in one process, {el1:.1f} s wall"}}


# ----------------------------------------------------------------- traffic records
def kernel_code_digest() -> str:
    """sha256 of the kernel source with comments and blank lines removed and
    whitespace collapsed: HBM counters recorded for one digest stay valid
    across comment edits, and are dropped once the code changes."""
    import hashlib
    import re
    src = (ROOT / "paged_kv_cache_438_amd" / "csrc" / "pa_kernels.hip").read_text()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    lines = [" ".join(re.sub(r"//.*", "", l).split()) for l in src.splitlines()]
    return hashlib.sha256("\n".join(l for l in lines if l).encode()).hexdigest()


# ----------------------------------------------------------------- block operations
def block_ops(args) -> dict:
    """Time pa_copy_blocks and pa_swap_blocks on blocks of the Llama-2-7B
    shape (32 KV heads x 16 tokens x 128 x fp16 = 128 KiB per block and
    pool).  Copies: 2048 seeded random (source, destination) pairs in an
    8192-block pool, bytes = read + write of K and V.  Swaps: 2048 blocks out
    to a pinned host pool and back in, once as runs of consecutive blocks
    (one copy per pool and run) and once scattered (one copy per block)."""
    import torch
    import paged_kv_cache_438_amd as pa
    if not pa.LIB_PATH.exists():
        raise SystemExit("libpa.so is not built: run python __graft_entry__.py build")
    Hkv, bs, d, NB, NP = 32, 16, 128, 8192, 2048
    block_bytes = Hkv * bs * d * 2
    rng = np.random.default_rng(7 if args.seed is None else args.seed)
    kp = torch.empty((NB, Hkv, bs, d), dtype=torch.float16, device="cuda").normal_()
    vp = torch.empty_like(kp).normal_()
    perm = rng.permutation(NB)
    pairs = np.stack([perm[:NP], perm[NP:2 * NP]], axis=1).astype(np.int32)
    dpairs = torch.from_numpy(pairs).cuda()
    hk = torch.empty((NP, Hkv, bs, d), dtype=torch.float16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    runs = [(int(perm[0] // NP) * NP + i, i) for i in range(NP)]      # consecutive blocks
    runs = [(g % NB, c) for g, c in runs]
    scattered = [(int(g), i) for i, g in enumerate(perm[:NP])]

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3

    reps = max(1, min(args.steps, 20))
    t_copy = timed(lambda: pa.pa_copy_blocks(kp, vp, dpairs), reps)
    copy_bytes = 2 * 2 * NP * block_bytes
    res = {"metric": "block copy / swap throughput", "unit": "GB/s", "n_gpus": 1,
           "data": "synthetic", "dtype": "f16",
           "config": {"workload": "llama2_7b blocks", "block_bytes_per_pool": block_bytes,
                      "pairs": NP, "pool_blocks": NB},
           "copy_blocks": {"us": round(t_copy * 1e6, 2),
                           "GBps": round(copy_bytes / t_copy / 1e9, 1),
                           "frac_of_8TBps": round(copy_bytes / t_copy / 8e12, 4),
                           "bytes": copy_bytes}}
    swap_bytes = 2 * NP * block_bytes
    for name, prs in (("consecutive", runs), ("scattered", scattered)):
        back = [(c, g) for g, c in prs]
        t_out = timed(lambda: pa.pa_swap_blocks(hk, hv, kp, vp, prs), max(1, reps // 4))
        t_in = timed(lambda: pa.pa_swap_blocks(kp, vp, hk, hv, back), max(1, reps // 4))
        res[f"swap_{name}"] = {"out_us": round(t_out * 1e6, 1),
                               "out_GBps": round(swap_bytes / t_out / 1e9, 2),
                               "in_us": round(t_in * 1e6, 1),
                               "in_GBps": round(swap_bytes / t_in / 1e9, 2),
                               "bytes": swap_bytes}
    print(json.dumps(res), flush=True)
    return 0


def read_ceiling(pa, torch, seed: int = 5) -> dict:
    """The read rate a decode kernel can approach on this GPU: pa_read_probe
    over a 1 GiB buffer in 4 KiB tiles (the size of one (block, head) tile at
    block_size 16, head_dim 128, 2-byte elements), read in order and in a
    seeded random order, plus the best pattern a tile-size sweep found (32 KiB
    tiles in order), 10 launches each, timed with HIP events."""
    total = 1 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    res = {"kind": "pa_read_probe over 1 GiB with non-temporal 16-byte loads: 4 KiB tiles "
                   "in order and in random order, 32 KiB tiles in order"}
    n4 = total // 4096
    cases = {"sequential": (4096, np.arange(n4, dtype=np.int32)),
             "random_tiles": (4096, np.random.default_rng(seed).permutation(n4).astype(np.int32)),
             "sequential_32KiB": (32768, np.arange(total // 32768, dtype=np.int32))}
    for name, (tile, order) in cases.items():
        o = torch.from_numpy(order).cuda()
        for _ in range(3):
            pa.pa_read_probe(buf, tile, o, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            pa.pa_read_probe(buf, tile, o, sink)
        b.record()
        torch.cuda.synchronize()
        res[name + "_GBps"] = round(total / (a.elapsed_time(b) / 10 * 1e-3) / 1e9, 1)
    del buf
    # The runtime's own figures: bus width and peak memory clock.  MI355X
    # reports 8192 bits at 2.0 GHz; its HBM3E pins run at about 8 Gb/s, i.e.
    # 4 transfers per reported clock, which implies 8.19 TB/s (the roofline
    # uses the published 8 TB/s).
    bw_bits, clk_khz = pa.pa_device_memory(torch.cuda.current_device())
    res["device_reported"] = {"bus_width_bits": bw_bits, "mem_clock_khz": clk_khz,
                              "transfers_per_clock": 4,
                              "implied_peak_GBps": round(4 * clk_khz * 1e3 * bw_bits / 8 / 1e9, 1)}
    return res


def read_sweep(seed: int = 5) -> int:
    """Tile-size sweep of pa_read_probe over a 1 GiB buffer: tiles of 4 to
    64 KiB, read in order and in a seeded random order, 10 launches each."""
    import torch
    import paged_kv_cache_438_amd as pa
    if not pa.LIB_PATH.exists():
        raise SystemExit("libpa.so is not built: run python __graft_entry__.py build")
    total = 1 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(seed)
    rows = []
    for tile in (4096, 8192, 16384, 32768, 65536):
        n = total // tile
        rec = {"tile_bytes": tile}
        for name, order in (("in_order", np.arange(n, dtype=np.int32)),
                            ("random", rng.permutation(n).astype(np.int32))):
            o = torch.from_numpy(order).cuda()
            for _ in range(3):
                pa.pa_read_probe(buf, tile, o, sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(10):
                pa.pa_read_probe(buf, tile, o, sink)
            b.record()
            torch.cuda.synchronize()
            rec[name + "_GBps"] = round(total / (a.elapsed_time(b) / 10 * 1e-3) / 1e9, 1)
        rows.append(rec)
    print(json.dumps({"metric": "pa_read_probe read rate by tile size", "unit": "GB/s",
                      "buffer_bytes": total, "rows": rows}), flush=True)
    return 0


# ----------------------------------------------------------------- GPU run
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama2_7b", choices=sorted(WORKLOADS))
    ap.add_argument("--entry", default=None, choices=["single", "splitk", "shared"])
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true",
                    help="do not compare the timed output with the oracle (profiler runs)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the workload's block size (page-size sweep)")
    ap.add_argument("--contiguous", action="store_true",
                    help="decode over a contiguous cache that reserves the workload's longest "
                         "possible context for every sequence, with no block table "
                         "(pa_decode_contiguous): the scheme the pages contrast paging with")
    ap.add_argument("--through-table", action="store_true",
                    help="with --contiguous: the paged entry over the same contiguous memory, "
                         "seen as one block per sequence through an identity table (isolates "
                         "the cost of the table lookups)")
    ap.add_argument("--shuffled", action="store_true",
                    help="with --through-table: the sequences' regions moved to shuffled "
                         "slots of the same memory, the table naming each one's slot")
    ap.add_argument("--one-block", action="store_true",
                    help="paged decode with one block per sequence, as long as the longest "
                         "possible sequence")
    ap.add_argument("--cached", action="store_true",
                    help="plain cached K/V loads (the shared-blocks policy) even without sharing")
    ap.add_argument("--valu-only", action="store_true",
                    help="grouped heads on the vector ALUs instead of the matrix cores")
    ap.add_argument("--separate-write", action="store_true",
                    help="paged pool: write the new token with pa_cache_write and time the "
                         "decode call alone, instead of the default single call "
                         "(pa_write_decode, pa_write_decode_splitk or "
                         "pa_write_decode_shared_prefix) timed as the whole step")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph after the warm-up and replay it for "
                         "the timed steps (the step's launches, nothing else)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the read-probe measurement reported beside the roofline")
    ap.add_argument("--block-ops", action="store_true",
                    help="instead of decode, time the block copy (copy-on-write) and swap "
                         "operations on the Llama-2-7B-shaped pool")
    ap.add_argument("--read-sweep", action="store_true",
                    help="instead of decode, sweep the read probe over tile sizes and orders")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the benchmark, run torch copies of this many MiB "
                         "(calibrates HBM byte counters under rocprofv3 --pmc)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): paged decode shards by sequence or KV head with no exchange inside "
              "attention, and this benchmark measures the single-GPU kernel.", flush=True)
        return 2

    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)
        return 0

    if args.block_ops:
        return block_ops(args)
    if args.read_sweep:
        return read_sweep()

    w = WORKLOADS[args.workload]
    entry, P = DEFAULT_ENTRY[w.name]
    longest = w.length_hi if w.length_kind != "shared_prefix" else w.prompt_len + w.length_hi
    if w.length_kind == "fixed":
        longest = max(w.lengths)
    if args.contiguous and (args.block_size or args.one_block or args.entry == "shared" or
                            (not args.entry and entry == "shared")):
        raise SystemExit("--contiguous runs the single-pass or split-K decode over its own "
                         "cache: no --block-size, --one-block or shared-prompt entry")
    if args.through_table and not (args.contiguous and longest & (longest - 1) == 0 and
                                   longest <= 65536):
        raise SystemExit("--through-table needs --contiguous and a longest context that is a "
                         "power of two of at most 65536 (a valid block size)")
    if args.shuffled and not args.through_table:
        raise SystemExit("--shuffled needs --through-table")
    if args.one_block or args.block_size:
        bs = args.block_size or 1 << (longest - 1).bit_length()
        if args.one_block and bs < longest:
            raise SystemExit("--one-block needs a block at least as long as the longest sequence")
        if w.length_kind == "shared_prefix" and w.prompt_len % bs:
            raise SystemExit("the shared prompt must be whole blocks")
        w = w.replace(block_size=bs, max_blocks_per_seq=-(-longest // bs))
    if args.entry:
        entry = args.entry
        P = args.partition or (w.partition_size or 1024) if entry != "single" else None
    elif args.partition:
        P = args.partition
    if args.separate_write and args.contiguous:
        raise SystemExit("--separate-write needs a paged pool (the contiguous cache's write "
                         "is always its own call)")
    # On a paged pool the step is one call by default.
    args.combined = not args.contiguous and not args.separate_write
    t = time.perf_counter()
    case = make_case(w, seed=args.seed, keep_logical=args.contiguous)
    log(f"bench: generated {w.name} seed={case.seed} in {time.perf_counter() - t:.1f} s; "
        f"sum L = {kv_token_count(case)}, pool blocks = {case.num_blocks}")

    # The oracle runs in fork pools before any GPU call.
    cpu, ref = None, None
    if not args.no_cpu_baseline:
        ref, cpu = cpu_baseline(case, args.cpu_seconds)
        log(f"bench: cpu baseline {cpu['value']:.4g} KV tokens/s on {cpu['cores']} workers")
    elif not args.no_check:
        ref = oracle_reference(case)

    import torch
    import paged_kv_cache_438_amd as pa
    if not pa.LIB_PATH.exists():
        raise SystemExit("libpa.so is not built: run python __graft_entry__.py build")
    dev = torch.device("cuda:0")

    def d(a, dt=None):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    dt = case.dtype
    q = d(case.q, dt)
    tb, ln = d(case.block_tables), d(case.context_lens)
    if args.contiguous:
        # Every sequence reserves the longest context the workload allows.
        kc, vc = contiguous_cache(case, longest, device=dev)
        case.logical_k = case.logical_v = None
        # The same memory as a pool of one block per sequence, block s for
        # sequence s; shuffled, sequence s's region moves to slot perm[s].
        ident = torch.arange(w.num_seqs, dtype=torch.int32, device=dev).reshape(-1, 1)
        if args.shuffled:
            perm = torch.from_numpy(np.random.default_rng(case.seed).permutation(w.num_seqs))
            perm = perm.to(dev)
            kc2, vc2 = torch.empty_like(kc), torch.empty_like(vc)
            kc2[perm], vc2[perm] = kc, vc
            kc, vc = kc2, vc2
            del kc2, vc2
            ident = perm.to(torch.int32).reshape(-1, 1).contiguous()
    else:
        kp, vp = d(case.k_pool, dt), d(case.v_pool, dt)
    kn, vn = d(case.k_new, dt), d(case.v_new, dt)
    out = torch.empty_like(q)
    maxlen = int(case.context_lens.max())
    scale = float(case.scale)
    ws = None
    if entry == "splitk":
        # A contiguous call bounds the partitions by its region length.
        bound = longest if args.contiguous else maxlen
        need = pa.pa_decode_splitk_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim, bound, P)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if entry == "shared":
        if case.shared_groups is None:
            raise SystemExit("--entry shared needs a workload with prompt groups")
        sg = np.full(w.num_seqs, -1, dtype=np.int32)
        for gi, members in enumerate(case.shared_groups):
            sg[members] = gi
        seq_group = d(sg)
        group_prefix = d(np.full(len(case.shared_groups), w.prompt_len, dtype=np.int32))
        max_group = int(case.shared_groups.shape[1])
        need = pa.pa_decode_shared_prefix_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim,
                                                          maxlen, P, len(case.shared_groups))
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

    # Cached K/V loads when several sequences' tables name the same blocks and
    # the kernel reads them once per sequence; the sharing-aware entry reads
    # a group's prompt once per KV head, so it streams.
    shared = args.cached or (case.shared_groups is not None and entry != "shared")

    def decode():
        if args.through_table and entry == "single":
            pa.pa_decode(q, kc, vc, ident, ln, scale=scale, out=out, valu_only=args.valu_only)
        elif args.through_table:
            pa.pa_decode_splitk(q, kc, vc, ident, ln, partition_size=P, max_context_len=longest,
                                scale=scale, out=out, workspace=ws, valu_only=args.valu_only)
        elif args.contiguous:
            pa.pa_decode_contiguous(q, kc, vc, ln, scale=scale, partition_size=P or 0, out=out,
                                    workspace=ws, valu_only=args.valu_only)
        elif entry == "single":
            pa.pa_decode(q, kp, vp, tb, ln, scale=scale, out=out, shared_kv=shared,
                         valu_only=args.valu_only)
        elif entry == "shared":
            pa.pa_decode_shared_prefix(q, kp, vp, tb, ln, seq_group, group_prefix, max_group, P,
                                       maxlen, scale=scale, out=out, workspace=ws,
                                       shared_kv=shared)
        else:
            pa.pa_decode_splitk(q, kp, vp, tb, ln, partition_size=P, max_context_len=maxlen,
                                scale=scale, out=out, workspace=ws, shared_kv=shared,
                                valu_only=args.valu_only)

    # A step is the new token's cache write and the decode.
    def write():
        if args.through_table:                  # the paged write through the same table
            pa.pa_cache_write(kc, vc, kn, vn, ident, ln)
        elif args.contiguous:
            pa.pa_cache_write_contiguous(kc, vc, kn, vn, ln)
        else:
            pa.pa_cache_write(kp, vp, kn, vn, tb, ln)

    # The same step as one call: the write runs in the plan's launch.
    def combined():
        if entry == "single":
            pa.pa_write_decode(q, kp, vp, kn, vn, tb, ln, scale=scale, out=out, shared_kv=shared,
                               valu_only=args.valu_only)
        elif entry == "shared":
            pa.pa_write_decode_shared_prefix(q, kp, vp, kn, vn, tb, ln, seq_group, group_prefix,
                                             max_group, P, maxlen, scale=scale, out=out,
                                             workspace=ws, shared_kv=shared)
        else:
            pa.pa_write_decode_splitk(q, kp, vp, kn, vn, tb, ln, partition_size=P,
                                      max_context_len=maxlen, scale=scale, out=out,
                                      workspace=ws, shared_kv=shared, valu_only=args.valu_only)

    def step():
        if args.combined:
            combined()
        else:
            write()
            decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        # Capture one step; the timed steps replay it.  The step's calls
        # allocate nothing and launch kernels only.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        step = graph.replay
    K = args.steps
    # The timed region: K steps back to back, HIP events on the launch
    # stream only at its two ends (an event between launches adds a few
    # microseconds to every step and to the launch it brackets).
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    span_ms = e0.elapsed_time(e1)
    if args.combined:
        # One call per step: the call's average duration is the span over K.
        dec_ms = span_ms / K
        timing = (f"events around the {K} timed steps, one call each" +
                  (", replayed from a HIP graph" if args.graph else ""))
    else:
        # Two calls per step: the decode alone, K more launches back to back
        # between two events, right after the timed region.
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        d0.record()
        for i in range(K):
            decode()
        d1.record()
        torch.cuda.synchronize()
        dec_ms = d0.elapsed_time(d1) / K
        timing = f"events around {K} back-to-back decode launches after the timed steps"

    e = w.elem_bytes
    # With prompt groups the blocks a group shares are counted once (unique
    # bytes, what HBM must deliver); the per-sequence sum is reported beside.
    # Table entries count only where a table is read (one per sequence
    # through the identity table).
    tables_read = not args.contiguous or args.through_table
    dec_bytes = algorithmic_bytes(case, unique=case.shared_groups is not None,
                                  tables=tables_read and not args.through_table)
    logical_bytes = algorithmic_bytes(case, tables=tables_read and not args.through_table)
    if args.through_table:
        dec_bytes += 4 * w.num_seqs
        logical_bytes += 4 * w.num_seqs
    # The write reads both new rows and writes them, plus the lengths and (paged) one table entry.
    cw_bytes = 4 * w.num_seqs * w.num_kv_heads * w.head_dim * e + \
        4 * (1 if args.contiguous and not args.through_table else 2) * w.num_seqs
    step_bytes = dec_bytes + cw_bytes
    ms_step = elapsed * 1e3 / K
    value = step_bytes * K / elapsed / 1e9
    tokens = kv_token_count(case)
    # The timed call: the decode, or (split entries, one call) the whole step.
    timed_bytes = step_bytes if args.combined else dec_bytes
    achieved = timed_bytes / (dec_ms * 1e-3) / 1e9

    # The output of the last timed step against the fp64 oracle, every
    # (sequence, head) row, within the storage dtype's max-abs bound.
    tol = TOLERANCE[dt]
    max_err = None
    if ref is not None:
        got = out.float().cpu().numpy().astype(np.float64)
        max_err = float(np.max(np.abs(got - ref))) if np.all(np.isfinite(got)) else float("inf")
        log(f"bench: timed output vs oracle: max|err| = {max_err:.3e} (bound {tol:.0e})")

    ceiling = read_ceiling(pa, torch) if not args.no_read_ceiling else None
    if ceiling:
        ceiling["decode_frac_of_random_tiles"] = round(achieved / ceiling["random_tiles_GBps"], 4)
        best = max(v for k, v in ceiling.items() if k.endswith("_GBps"))
        ceiling["decode_frac_of_best_read"] = round(achieved / best, 4)

    traffic = None
    entry_key = entry if args.through_table else "contiguous" if args.contiguous else entry
    if args.combined:
        entry_key += "_combined"
    tf = ROOT / "profiles" / f"traffic_{w.name}_{entry_key}.json"
    if tf.exists():
        try:
            rec = json.loads(tf.read_text())
            if rec.get("kernel_code_sha256") == kernel_code_digest():
                traffic = rec.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    mfma = entry == "shared" or (dt != "f32" and w.group_ratio >= 2 and not args.valu_only)
    kname = "k_decode_mfma" if mfma else "k_decode"
    kernel = kname if not P else f"k_plan + {kname} (partitions) + k_reduce"
    if args.combined and not P:
        # the vector kernel with one query head per workgroup (odd group), big pages
        fused = not mfma and w.group_ratio % 2 == 1 and w.block_size >= 16 and not shared
        kernel = (f"{kname} (with the new-token write)" if fused
                  else f"k_cache_write + {kname}")
    elif args.combined:
        kernel = f"k_write_plan (new-token write + plan) + {kname} (partitions) + k_reduce"
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "f16": "f16", "bf16": "bf16"}[dt],
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "seed": case.seed,
                   "block_size": longest if args.through_table else None if args.contiguous
                   else w.block_size,
                   "max_len": longest if args.contiguous else None,
                   "entry": ENTRY_NAME[entry_key],
                   "partition_size": P, "accumulate": "f32", "shared_kv_flag": shared,
                   "valu_only": bool(args.valu_only), "hip_graph": bool(args.graph),
                   "global_batch": w.num_seqs, "kv_tokens": tokens,
                   "kv_layout": ("contiguous cache, regions shuffled, through a table"
                                 if args.shuffled else
                                 "contiguous cache through an identity table"
                                 if args.through_table else "contiguous cache"
                                 if args.contiguous else "paged pool"),
                   "step": "pa_cache_write_contiguous + decode"
                   if args.contiguous and not args.through_table
                   else ENTRY_NAME[entry_key] + " (write and decode in one call)"
                   if args.combined else "pa_cache_write + decode",
                   "parallelism": "none (1 GPU)"},
        "max_abs_err": max_err,
        "tolerance": tol,
        "check": ("output of the last timed step vs the fp64 oracle, all "
                  f"{w.num_seqs * w.num_heads} (sequence, head) rows") if ref is not None
                 else "skipped (--no-check)",
        # Share of the reserved KV memory that holds tokens: used blocks over
        # the pool, or tokens over the rows a contiguous cache reserves.
        "pool_utilization": round(tokens / (w.num_seqs * longest) if args.contiguous
                                  else case.unique_blocks / case.num_blocks, 4),
        "kv_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "avg_launch_us": round(dec_ms * 1e3, 3),
                     "timing": timing,
                     "step_span_us": round(span_ms * 1e3 / K, 3),
                     "algorithmic_bytes_per_launch": timed_bytes,
                     "logical_bytes_per_launch": logical_bytes},
        "cpu_baseline": cpu,
        "read_ceiling": ceiling,
    }
    print(json.dumps(res), flush=True)
    if max_err is not None and not max_err <= tol:
        log(f"bench: FAILED: timed output differs from the oracle by {max_err} > {tol}")
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
