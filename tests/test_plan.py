"""mla_decode_plan (host): the length-proportional work list of the ragged decode.

Checked on the properties its header states: every sequence's units are
consecutive, page-aligned and cover [0, L) exactly once; unit lengths stay at or
below the unit length U, the fewest whole pages whose unit count is within the
target (one page less would exceed it); the count is padded to a multiple of 8
with empty units that no sequence's range holds; argument errors return the
stated statuses."""
import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
from mla_latent_kv_dkv_amd import inputs as I


def _check_plan(lens, page, target):
    lens = np.asarray(lens, dtype=np.int32)
    n, plan = M.mla_decode_plan(lens, page, target)
    B = len(lens)
    assert n >= 8 and n % 8 == 0
    units = plan[:3 * n].reshape(n, 3)
    start = plan[3 * n:]
    assert len(start) == B + 1 and start[0] == 0
    count = lambda u: sum(max(1, -(-int(L) // u)) for L in lens)
    top = max(1, -(-int(lens.max()) // page))               # pages of the longest sequence
    pages = next((p for p in range(1, top + 1) if count(p * page) <= target), top)
    U = pages * page
    if pages > 1 and count(U) <= target:
        assert count(U - page) > target                   # the fewest pages that fit
    for b in range(B):
        mine = units[start[b]:start[b + 1]]
        assert len(mine) >= 1
        assert (mine[:, 0] == b).all()
        if lens[b] == 0:
            assert len(mine) == 1 and mine[0, 1] == 0 and mine[0, 2] == 0
            continue
        assert mine[0, 1] == 0 and mine[-1, 2] == lens[b]
        assert (mine[1:, 1] == mine[:-1, 2]).all()          # contiguous
        assert (mine[:, 1] < mine[:, 2]).all()              # no empty unit
        assert (mine[:, 1] % page == 0).all()               # page-aligned starts
        assert (mine[:, 2] - mine[:, 1] <= U).all()
        assert len(mine) == max(1, -(-int(lens[b]) // U))
    assert start[B] <= max(target, B)
    pad = units[start[B]:]
    assert (pad == 0).all()
    return n, units, start


def test_plan_ragged_workload():
    w = I.WORKLOADS["ragged"]
    lens = I.seq_lengths(w)
    n, units, start = _check_plan(lens, 64, 768)
    # within the target and close to it, and the longest sequence split the most
    assert 0.9 * 768 <= start[-1] <= 768
    counts = np.diff(start)
    assert counts[np.argmax(lens)] == counts.max() and counts[np.argmin(lens)] == 1


@pytest.mark.parametrize("lens,page,target", [
    ([1], 64, 1), ([64], 64, 8), ([65], 64, 8), ([0, 0, 5], 16, 3), ([4096] * 64, 64, 256),
    ([131072] * 4, 64, 256), ([7, 1000, 33, 0, 4097], 16, 40), ([100] * 3, 1, 7)])
def test_plan_properties(lens, page, target):
    _check_plan(lens, page, target)


def test_plan_uniform_lengths_match_the_split_rule():
    """Equal lengths with target = batch x S give S units per sequence at the
    uniform split's boundaries (the same page-aligned chunk rule)."""
    import oracle as O
    L, B, S = 4096, 8, 4
    n, units, start = _check_plan([L] * B, 64, B * S)
    for b in range(B):
        got = [(int(t0), int(t1)) for _, t0, t1 in units[start[b]:start[b + 1]]]
        assert got == [(a, e) for a, e in O.split_bounds(L, S, 64) if a < e]


def test_plan_errors():
    lib = M.load()
    import ctypes
    lens = np.array([10, 20], dtype=np.int32)
    cap = M.mla_decode_plan_capacity(2, 4)
    out = np.zeros(cap, dtype=np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.mla_decode_plan(None, 2, 64, 4, P(out), cap) == -1
    assert lib.mla_decode_plan(P(lens), 2, 64, 4, None, cap) == -1
    assert lib.mla_decode_plan(P(lens), 0, 64, 4, P(out), cap) == -2
    assert lib.mla_decode_plan(P(lens), 2, 0, 4, P(out), cap) == -2
    assert lib.mla_decode_plan(P(lens), 2, 64, 0, P(out), cap) == -2
    assert lib.mla_decode_plan(P(lens), 2, 64, 4, P(out), cap - 1) == -4
    bad = np.array([10, -1], dtype=np.int32)
    assert lib.mla_decode_plan(P(bad), 2, 64, 4, P(out), cap) == -2
    assert M.mla_decode_plan_capacity(-1, 4) == 0
    assert lib.mla_decode_plan(P(lens), 2, 64, 4, P(out), cap) == 8


def test_plan_random_batches():
    """Seeded random ragged batches (empty sequences included, targets below and far
    above the batch size): every property above, and a count within the target
    whenever the batch alone does not exceed it."""
    rng = np.random.default_rng(20261204)
    for _ in range(40):
        B = int(rng.integers(1, 90))
        lens = rng.integers(0, 20000, size=B)
        lens[rng.random(B) < 0.1] = 0
        page = int(rng.choice([16, 64]))
        target = int(rng.integers(1, 1200))
        n, units, start = _check_plan(lens, page, target)
        if target >= B:
            assert start[-1] <= target
