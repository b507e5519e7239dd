"""Pins for the oracle planner (view, cost, LPT homes, params_by_home, offsets).

Each check compares the oracle with something other than itself: values
printed on the owner_planning page, costs worked out by hand, hand-traced LPT
cases, and Graham's LPT bound against an exhaustive search.
"""

import itertools
import json
import os
import random

import pytest

from oracle import planner

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_view_and_eligibility():
    # owner_planning page, select_ge_2d_params / ns_cost_fn view.
    assert planner.matrix_view((7,)) is None
    assert planner.matrix_view(()) is None
    assert planner.matrix_view((3, 5)) == (3, 5)
    assert planner.matrix_view((2, 3, 4)) == (2, 12)
    assert planner.matrix_view((4, 1, 1, 9)) == (4, 9)


def test_cost_hand_values():
    for case in _load("cost_hand_values.json")["cases"]:
        assert planner.ns_cost(case["shape"], case["steps"]) == case["cost"], case


def _costs(ks):
    # shape (1, k) with one step costs k * (1 + 1) = 2k: a handle on exact costs.
    return [(1, k) for k in ks]


def test_lpt_descending_on_two_homes():
    # costs 20, 14, 12, 10 (shapes (1,10),(1,7),(1,6),(1,5) at one step).
    # Traced by hand: 20 -> h0 [20,0]; 14 -> h1 [20,14]; 12 -> h1 [20,26];
    # 10 -> h0 [30,26].
    p = planner.plan(_costs([10, 7, 6, 5]), steps=1, num_homes=2)
    assert p["home"] == [0, 1, 1, 0]
    assert p["load"] == [30, 26]
    assert p["order"] == [0, 1, 2, 3]


def test_lpt_sorts_by_cost_not_index():
    # costs 2, 20, 12 -> order by descending cost: 1, 2, 0.
    # 20 -> h0; 12 -> h1; 2 -> h1 (12 < 20).
    p = planner.plan(_costs([1, 10, 6]), steps=1, num_homes=2)
    assert p["order"] == [1, 2, 0]
    assert p["home"] == [1, 0, 1]
    assert p["load"] == [20, 14]


def test_lpt_ties_follow_buffer_order():
    # four equal costs on three homes: ties go to the first candidate.
    p = planner.plan(_costs([3, 3, 3, 3]), steps=1, num_homes=3)
    assert p["home"] == [0, 1, 2, 0]
    # equal loads, candidates restricted to homes 1 and 2 -> home 1.
    p = planner.plan(_costs([4]), steps=1, num_homes=3, split_rows=[[0, 1, 0]])
    assert p["home"] == [1]
    p = planner.plan([(2, 4)], steps=1, num_homes=3, split_rows=[[0, 1, 1]])
    assert p["home"] == [1]


def test_lpt_single_candidate_first():
    # tensor 0 is big and may go anywhere; tensor 1 is small and only home 0
    # holds it. Single-candidate tensors are placed first, so tensor 1 takes
    # home 0 and tensor 0 then goes to the empty home 1. (Placing by cost
    # alone would put both on home 0.)
    shapes = [(2, 50), (2, 3)]
    split = [[1, 1], [2, 0]]
    p = planner.plan(shapes, steps=1, num_homes=2, split_rows=split)
    assert p["home"] == [1, 0]
    assert p["order"] == [1, 0]


def test_lpt_no_candidate_is_error():
    with pytest.raises(ValueError):
        planner.plan([(0, 5)], steps=5, num_homes=2, split_rows=[[0, 0]])
    with pytest.raises(ValueError):
        planner.plan([(4, 5)], steps=5, num_homes=2, split_rows=[[1, 2]])  # sums to 3 != 4


def test_ineligible_tensors_skipped():
    p = planner.plan([(5,), (2, 3), (7,)], steps=5, num_homes=2)
    assert p["home"] == [-1, 0, -1]
    assert p["cost"] == [0, 6 * (2 * 5 + 1), 0]
    assert p["order"] == [1]


def test_worked_example_default_balancer():
    ex = _load("owner_gather_example.json")
    shapes = ex["printed"]["shapes"]
    split = ex["derived_by_hand"]["split_rows"]
    # the split rows are the first dims of the printed local shard shapes
    pr = ex["printed"]["local_shard_shapes"]
    assert split == [[pr["rank0"][0][0], pr["rank1"][0][0]], [pr["rank0"][1][0], pr["rank1"][1][0]]]
    p = planner.plan(shapes, steps=5, num_homes=2, split_rows=split)
    d = ex["derived_by_hand"]
    assert p["home"] == d["default_balancer_owners"]
    assert p["load"] == d["default_balancer_loads"]
    assert p["order"] == d["default_balancer_order"]
    assert p["home"] != [ex["printed"]["tensor_to_owner"]["0"], ex["printed"]["tensor_to_owner"]["1"]]


def test_graham_bound_exhaustive():
    """LPT makespan <= (4/3 - 1/(3S)) * OPT (Graham 1969) on tiny sets, OPT by brute force."""
    rng = random.Random(1234)
    worst = 0.0
    for _ in range(300):
        S = rng.randint(2, 3)
        n = rng.randint(1, 7)
        ks = [rng.randint(1, 40) for _ in range(n)]
        costs = [2 * k for k in ks]
        p = planner.plan(_costs(ks), steps=1, num_homes=S)
        lpt = max(p["load"])
        assert sum(p["load"]) == sum(costs)
        opt = min(max(sum(c for c, h in zip(costs, assign) if h == s) for s in range(S))
                  for assign in itertools.product(range(S), repeat=n))
        bound = (4.0 / 3.0 - 1.0 / (3.0 * S)) * opt
        assert lpt <= bound + 1e-9, (ks, S, p, opt)
        worst = max(worst, lpt / bound)
    assert worst <= 1.0


def test_params_by_home_worked_example():
    assert planner.params_by_home(2, [1, 1], 2) == [[], [0, 1]]
    assert planner.params_by_home(4, [2, 0, 2, 0], 3) == [[1, 3], [], [0, 2]]
    with pytest.raises(ValueError):
        planner.params_by_home(1, [3], 2)


def test_route_offsets_worked_example():
    ex = _load("owner_gather_example.json")
    d = ex["derived_by_hand"]
    shapes = ex["printed"]["shapes"]
    owners = [ex["printed"]["tensor_to_owner"]["0"], ex["printed"]["tensor_to_owner"]["1"]]
    off = planner.route_offsets(shapes, d["split_rows"], owners, 2)
    assert off["shard_elems"] == d["shard_elems"]
    # rank ranges [0,20) and [20,40) of the page: each shard holds 20 elements
    assert off["shard_elems"] == [r[1] - r[0] for r in ex["printed"]["rank_ranges"]]
    assert off["shard_offset"] == d["shard_offset"]
    assert off["row_start"] == d["row_start"]
    assert off["home_offset"] == d["home_offset_for_owners_1_1"]
    assert off["home_elems"] == d["home_elems_for_owners_1_1"]
    # rank 0 sends 20 elements of param_0 to owner 1, starting at offset 0 of its buffer
    assert off["shard_offset"][0][0] == ex["printed"]["rank1_recv_offsets"][0]["offset"]
    assert d["split_rows"][0][0] * 4 == ex["printed"]["rank0_send_buffer_elems_to_owner1"]
    assert ex["printed"]["layout_size"] == sum(off["home_elems"])


def test_wave_plan_page_example_and_hand_cases():
    # issue page, "Current Progress": 3000 tensors on 1000 slots -> 3 waves.
    shapes = [(8, 8)] * 3000
    wave, num = planner.wave_plan(shapes, 1000)
    assert num == 3
    assert [wave.count(w) for w in range(3)] == [1000, 1000, 1000]
    # default ready order is reverse index order: the last 1000 tensors go first
    assert wave[2999] == 0 and wave[2000] == 0 and wave[1999] == 1 and wave[0] == 2
    # more slots than tensors: one wave
    assert planner.wave_plan([(2, 2)] * 5, 8) == ([0] * 5, 1)
    # a caller-given order, and tensors with < 2 dims left out (no slot used)
    w, n = planner.wave_plan([(3, 3), (4,), (2, 5), (6, 1), (7,)], 2, ready_order=[0, 1, 2, 3, 4])
    assert (w, n) == ([0, -1, 0, 1, -1], 2)
    assert planner.wave_plan([], 3) == ([], 0)
    assert planner.wave_plan([(5,)], 3) == ([-1], 0)


@pytest.mark.parametrize("seed", range(10))
def test_wave_plan_counting_identities(seed):
    rng = random.Random(500 + seed)
    n = rng.randint(0, 60)
    shapes = [tuple(rng.randint(1, 9) for _ in range(rng.choice([1, 2, 3]))) for _ in range(n)]
    slots = rng.randint(1, 12)
    order = list(range(n))
    rng.shuffle(order)
    wave, num = planner.wave_plan(shapes, slots, order)
    eligible = [i for i in order if len(shapes[i]) >= 2]
    assert num == -(-len(eligible) // slots)
    # every wave but the last is full, waves are consecutive runs of the order
    for w in range(num):
        members = [i for i in eligible if wave[i] == w]
        assert len(members) == (slots if w < num - 1 else len(eligible) - slots * (num - 1))
        assert members == eligible[w * slots:w * slots + len(members)]
    assert all(wave[i] == -1 for i in range(n) if len(shapes[i]) < 2)
