"""CPU tests: the block-copy and block-swap oracle against its pins, and
planted mistakes in it caught by those pins.

Pins: a hand-typed 4-block fixture (tests/golden/block_ops_example.json),
decode through a privately copied block equalling decode through the shared
original (copy-on-write must be invisible to attention, "Efficient Memory
Management ... paper summary", key feature 2), and a swap out to CPU blocks
and back into other GPU blocks leaving decode bit-identical ("vLLM's
efficiency secret ...", section "Dynamic memory management")."""
from __future__ import annotations

import json
import pathlib

import numpy as np
import pytest

import oracle
import oracle.block_ops as BO
from tests.pins import random_tiny_case

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _fixture():
    fx = json.loads((GOLDEN / "block_ops_example.json").read_text())
    a = lambda x: np.array(x, dtype=np.float32)
    return fx, a(fx["k_pool"]), a(fx["v_pool"]), a


def pin_fixture(M):
    fx, kp, vp, a = _fixture()
    k2, v2 = M.copy_blocks(kp, vp, fx["copy"]["pairs"])
    assert np.array_equal(k2, a(fx["copy"]["expected_k"]))
    assert np.array_equal(v2, a(fx["copy"]["expected_v"]))
    assert np.array_equal(kp, a(fx["k_pool"]))          # inputs untouched
    so = fx["swap_out"]
    ck = np.zeros((so["cpu_blocks"],) + kp.shape[1:], dtype=np.float32)
    cv = np.zeros_like(ck)
    hk, hv = M.swap_blocks(ck, cv, kp, vp, so["pairs"])
    assert np.array_equal(hk, a(so["expected_k"]))
    assert np.array_equal(hv, a(so["expected_v"]))


def pin_copy_is_invisible_to_decode(M):
    for seed in range(4):
        rng = np.random.default_rng(300 + seed)
        dtype = ("f32", "f16", "bf16", "f16")[seed]
        bs = (1, 2, 4, 16)[seed]
        q, kp, vp, tb, lens, scale, _, _ = random_tiny_case(rng, 3, 30, bs, 4, 2, 2, dtype)
        lens[0] = max(int(lens[0]), 1)
        nb0 = -(-int(lens[0]) // bs)
        if tb[0, nb0 - 1] < 0:
            continue
        # three extra free blocks; copy seq 0's last block and its first into two of them
        pad = np.full((3,) + kp.shape[1:], kp.flat[0], dtype=kp.dtype)
        kp2, vp2 = np.concatenate([kp, pad]), np.concatenate([vp, pad])
        NB = kp.shape[0]
        pairs = [(int(tb[0, nb0 - 1]), NB), (int(tb[0, 0]), NB + 2)] if nb0 > 1 else \
                [(int(tb[0, 0]), NB + 2)]
        kc, vc = M.copy_blocks(kp2, vp2, pairs)
        tb2 = tb.copy()
        for src, dst in pairs:
            tb2[0, list(tb[0]).index(src)] = dst
        ref = oracle.decode(q, kp2, vp2, tb, lens, scale, bs, dtype)
        got = oracle.decode(q, kc, vc, tb2, lens, scale, bs, dtype)
        assert np.array_equal(ref, got, equal_nan=True), seed


def pin_swap_round_trip(M):
    rng = np.random.default_rng(9)
    q, kp, vp, tb, lens, scale, _, _ = random_tiny_case(rng, 4, 40, 4, 8, 2, 1, "f16")
    used = sorted({int(b) for s in range(4) for b in tb[s, :-(-int(lens[s]) // 4)]})
    NB, NC = kp.shape[0], len(used) + 2
    cpu_k = np.zeros((NC,) + kp.shape[1:], dtype=kp.dtype)
    cpu_v = np.zeros_like(cpu_k)
    out_pairs = [(b, i + 1) for i, b in enumerate(used)]
    ck, cv = M.swap_blocks(cpu_k, cpu_v, kp, vp, out_pairs)
    # back into a larger pool, each block at a new place
    big_k = np.zeros((NB + len(used),) + kp.shape[1:], dtype=kp.dtype)
    big_v = np.zeros_like(big_k)
    dest = {b: NB + i for i, b in enumerate(used)}
    gk, gv = M.swap_blocks(big_k, big_v, ck, cv, [(i + 1, dest[b]) for i, b in enumerate(used)])
    tb2 = np.where(tb >= 0, np.vectorize(lambda x: dest.get(int(x), -1))(tb), -1).astype(np.int32)
    ref = oracle.decode(q, kp, vp, tb, lens, scale, 4, "f16")
    got = oracle.decode(q, gk, gv, tb2, lens, scale, 4, "f16")
    assert np.array_equal(ref, got)
    for b in used:
        assert gk[dest[b]].tobytes() == kp[b].tobytes()
        assert gv[dest[b]].tobytes() == vp[b].tobytes()


def pin_refusals(M):
    fx, kp, vp, _ = _fixture()
    with pytest.raises(ValueError):
        M.swap_blocks(kp, vp, kp, vp, [(4, 0)])           # source outside the pool
    with pytest.raises(ValueError):
        M.copy_blocks(kp, vp, [(0, 1), (2, 1)])           # one destination twice
    with pytest.raises(ValueError):
        M.copy_blocks(kp, vp, [(0, 1), (1, 2)])           # a destination that is a source


PINS = [pin_fixture, pin_copy_is_invisible_to_decode, pin_swap_round_trip, pin_refusals]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_block_ops_pin(pin):
    pin(BO)


# ------------------------------------------------------------ planted mistakes
class _Mutant:
    copy_blocks = staticmethod(BO.copy_blocks)
    swap_blocks = staticmethod(BO.swap_blocks)


def _copy_reversed(k, v, pairs):
    return BO.copy_blocks(k, v, [(d, s) for s, d in BO._pair_list(pairs)])


def _copy_k_only(k, v, pairs):
    k2, _ = BO.copy_blocks(k, v, pairs)
    return k2, v.copy()


def _copy_head_axis(k, v, pairs):
    k2, v2 = k.copy(), v.copy()
    for s, d in BO._pair_list(pairs):
        if 0 <= s < k.shape[1] and 0 <= d < k.shape[1] and s != d:
            k2[:, d], v2[:, d] = k[:, s], v[:, s]
    return k2, v2


def _copy_first_head_only(k, v, pairs):
    k2, v2 = k.copy(), v.copy()
    full_k, full_v = BO.copy_blocks(k, v, pairs)
    k2[:, 0], v2[:, 0] = full_k[:, 0], full_v[:, 0]
    return k2, v2


def _swap_into_source(dk, dv, sk, sv, pairs):
    dk2, dv2 = BO.swap_blocks(dk, dv, sk, sv, [])
    for s, d in BO._pair_list(pairs):
        if d < sk.shape[0] and s < dk.shape[0]:
            dk2[s] = sk[d]
            dv2[s] = sv[d]
    return dk2, dv2


MUTANTS = [("copy_blocks", _copy_reversed), ("copy_blocks", _copy_k_only),
           ("copy_blocks", _copy_head_axis), ("copy_blocks", _copy_first_head_only),
           ("swap_blocks", _swap_into_source)]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m[1].__name__)
def test_planted_block_op_mistake_is_caught(mutant):
    name, fn = mutant
    M = type("M", (_Mutant,), {name: staticmethod(fn)})
    failed = 0
    for pin in PINS:
        try:
            pin(M)
        except (AssertionError, ValueError, IndexError, pytest.fail.Exception):
            failed += 1
    assert failed >= 1, f"no pin catches {fn.__name__}"
