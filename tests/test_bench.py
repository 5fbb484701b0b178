"""The benchmark's contract: one JSON line with the metric, the timing, the
roofline record and the baseline fields (GPU), and a plain refusal for more
than one GPU (CPU)."""
from __future__ import annotations

import json
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stdout


@pytest.mark.parametrize("args", [("--through-table",),
                                  ("--contiguous", "--through-table", "--workload", "tiny"),
                                  ("--contiguous", "--one-block"),
                                  ("--contiguous", "--workload", "shared_prefix"),
                                  ("--separate-write", "--contiguous"),
                                  ("--separate-write", "--contiguous", "--entry", "splitk")])
def test_layout_options_that_do_not_combine_are_refused(args):
    """Refused before any input is generated or the GPU is touched."""
    r = _bench(*args)
    assert r.returncode == 1
    assert "needs" in r.stderr or "runs the single-pass" in r.stderr, r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("args", [("--workload", "tiny"),
                                  ("--workload", "tiny", "--entry", "splitk", "--partition", "16"),
                                  ("--workload", "tiny", "--contiguous"),
                                  ("--workload", "tiny", "--contiguous", "--entry", "splitk",
                                   "--partition", "16"),
                                  ("--workload", "tiny", "--entry", "splitk", "--partition", "16",
                                   "--separate-write"),
                                  ("--workload", "tiny", "--separate-write"),
                                  ("--workload", "tiny", "--entry", "splitk", "--partition", "16",
                                   "--graph")])
def test_bench_prints_one_json_line(args):
    r = _bench(*args, "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "max_abs_err", "tolerance", "pool_utilization"):
        assert key in rec, key
    assert rec["max_abs_err"] is not None and rec["max_abs_err"] <= rec["tolerance"] == 1e-5
    assert 0.0 < rec["pool_utilization"] <= 1.0
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"] == "tiny"
    rf = rec["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


@pytest.mark.gpu
def test_block_ops_mode_prints_one_json_line():
    r = _bench("--block-ops", "--steps", "2")
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    assert rec["copy_blocks"]["GBps"] > 0
    assert rec["swap_consecutive"]["out_GBps"] > 0 and rec["swap_scattered"]["in_GBps"] > 0


def test_cpu_baseline_record_on_the_tiny_workload():
    """The oracle's timing record: pool rate, worker count and the
    single-process rate, on whole passes of the workload."""
    import importlib.util
    sys.path.insert(0, str(ROOT))
    from synthetic import TINY, kv_token_count, make_case
    spec = importlib.util.spec_from_file_location("bench_mod", ROOT / "bench.py")
    bench = importlib.util.module_from_spec(spec)
    sys.modules["bench_mod"] = bench          # the fork pool pickles its worker by name
    spec.loader.exec_module(bench)
    import numpy as np
    import oracle
    case = make_case(TINY)
    ref, rec = bench.cpu_baseline(case, 0.2)
    # the pass's rows, put back in sequence order, are the oracle's output
    full = oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables, case.context_lens,
                         case.scale, case.block_size, case.dtype)
    assert np.array_equal(ref, full)
    assert np.array_equal(bench.oracle_reference(case), full)
    assert rec["kind"] == "oracle" and rec["unit"] == "KV tokens/s"
    assert rec["value"] > 0 and 1 <= rec["cores"] <= 16
    assert str(kv_token_count(case)) in rec["sample"]
    one = rec["one_worker"]
    assert one["cores"] == 1 and one["value"] > 0


@pytest.mark.gpu
def test_read_sweep_mode_prints_one_json_line():
    r = _bench("--read-sweep")
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    assert [x["tile_bytes"] for x in rec["rows"]] == [4096, 8192, 16384, 32768, 65536]
    assert all(x["in_order_GBps"] > 0 and x["random_GBps"] > 0 for x in rec["rows"])
