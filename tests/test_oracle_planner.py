"""Pins for the oracle planners (CPU only).

Pinned against: hand-worked plans (tests/golden/plan_tiny.txt),
numpy.array_split on the tile indices (a library routine), and invariants
that any correct plan must satisfy (exactly-once coverage, balance).
"""

import os

import numpy as np
import pytest

from oracle.planner import plan_dynamic, plan_static

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_tiny.txt")
TINY = [17, 64, 200, 513]


def load_golden():
    plans, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "plan":
            cur = {"kind": f[1], "args": [int(x) for x in f[2:]], "items": []}
        elif f[0] == "item":
            cur["items"].append(tuple(int(x) for x in f[1:]))
        elif f[0] == "end":
            plans.append(cur)
        else:
            cur[f[0]] = [int(x) for x in f[1:]]
    return plans


def flat(g):
    out = list(g["header"]) + list(g["wg_ptr"])
    for it in g["items"]:
        out += list(it)
    return out + list(g["req_part_ptr"])


@pytest.mark.parametrize("g", load_golden(), ids=lambda g: f"{g['kind']}{g['args']}")
def test_golden_tiny(g):
    if g["kind"] == "dynamic":
        p = plan_dynamic(TINY, *g["args"])
    else:
        p = plan_static(TINY, *g["args"])
    assert p.items == g["items"]
    assert p.wg_ptr == g["wg_ptr"]
    assert p.req_part_ptr == g["req_part_ptr"]
    assert p.to_list() == flat(g)


def tiles_of(lens, tile_len):
    return [(b, j) for b, L in enumerate(lens) for j in range(-(-L // tile_len))]


def check_coverage(p, lens):
    """Items of each request tile [0, len_b) exactly once, in order."""
    for b, L in enumerate(lens):
        its = sorted((k0, k1) for (bb, k0, k1, _) in p.items if bb == b)
        assert its[0][0] == 0 and its[-1][1] == L
        for (a0, a1), (b0, b1) in zip(its, its[1:]):
            assert a1 == b0
        assert all(k1 > k0 for k0, k1 in its)


def check_slots(p, lens):
    n_items = [sum(1 for it in p.items if it[0] == b) for b in range(len(lens))]
    slots = [it[3] for it in p.items if it[3] >= 0]
    assert slots == list(range(len(slots)))             # numbered in item order
    for b in range(len(lens)):
        mine = [it[3] for it in p.items if it[0] == b]
        if n_items[b] == 1:
            assert mine == [-1]
        else:
            assert mine == list(range(p.req_part_ptr[b], p.req_part_ptr[b + 1]))


def random_lens(rng, B, lo, hi):
    return [int(x) for x in rng.integers(lo, hi + 1, size=B)]


@pytest.mark.parametrize("seed", range(40))
def test_dynamic_matches_array_split(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = random_lens(rng, B, 1, int(rng.choice([20, 300, 5000])))
    tile_len = int(rng.choice([1, 7, 16, 64, 128, 256]))
    W = int(rng.choice([1, 2, 5, 64, 300]))
    p = plan_dynamic(lens, tile_len, W)
    tiles = tiles_of(lens, tile_len)
    parts = np.array_split(np.arange(len(tiles)), W)
    assert p.n_tiles == len(tiles)
    for w in range(W):
        got = []
        for (b, k0, k1, _) in p.items[p.wg_ptr[w]:p.wg_ptr[w + 1]]:
            got += [(b, j) for j in range(k0 // tile_len, -(-k1 // tile_len))]
        assert got == [tiles[i] for i in parts[w]]
        # one item per request run
        bs = [it[0] for it in p.items[p.wg_ptr[w]:p.wg_ptr[w + 1]]]
        assert len(bs) == len(set(bs))
    check_coverage(p, lens)
    check_slots(p, lens)
    assert p.n_items <= W + B - 1


def test_dynamic_single_workgroup():
    lens = [5, 100, 1, 77]
    p = plan_dynamic(lens, 16, 1)
    assert p.items == [(b, 0, L, -1) for b, L in enumerate(lens)]
    assert p.req_part_ptr == [0] * 5


def test_dynamic_more_workgroups_than_tiles():
    lens = [30, 10]
    p = plan_dynamic(lens, 8, 50)
    for w in range(50):
        n = p.wg_ptr[w + 1] - p.wg_ptr[w]
        assert n == (1 if w < p.n_tiles else 0)


@pytest.mark.parametrize("S", [1, 2, 3, 8, 64])
def test_static_rule(S):
    rng = np.random.default_rng(S)
    lens = random_lens(rng, 17, 1, 300) + [1, 2, 3]
    p = plan_static(lens, S)
    assert p.n_workgroups == len(lens) * S and p.tile_len == 0
    for b, L in enumerate(lens):
        for c in range(S):
            w = b * S + c
            its = p.items[p.wg_ptr[w]:p.wg_ptr[w + 1]]
            lo, hi = c * L // S, (c + 1) * L // S
            assert its == ([] if hi == lo else [(b, lo, hi, its[0][3])])
    check_coverage(p, lens)
    check_slots(p, lens)


def test_invalid_arguments():
    for args in [([], 16, 4), ([0, 5], 16, 4), ([5], 0, 4), ([5], 16, 0)]:
        with pytest.raises(ValueError):
            plan_dynamic(*args)
    with pytest.raises(ValueError):
        plan_static([5], 0)
