"""Pins of the reference planner (oracle.plan): a hand-worked plan, LPT properties,
Graham's bound against brute-force optimal makespans, and hand-worked automatic
tile sizes. CPU only."""

import itertools
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import plan as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_invariants(seq_lens, Hkv, T, W, p):
    items = p["items"]
    B = len(seq_lens)
    nb = [(int(L) + T - 1) // T for L in seq_lens]
    assert list(p["req_tile_base"]) == list(np.concatenate([[0], np.cumsum(nb)]))
    seen = {(int(b), int(g), int(i)) for b, g, i, _ in items}
    assert len(seen) == len(items) == Hkv * sum(nb)
    assert seen == {(b, g, i) for b in range(B) for g in range(Hkv) for i in range(nb[b])}
    slots = sorted(int(s) for *_, s in items)
    assert slots == list(range(len(items)))
    for b, g, i, s in items:
        assert s == Hkv * p["req_tile_base"][b] + g * nb[b] + i
    assert p["worker_offsets"][0] == 0 and p["worker_offsets"][-1] == len(items)
    assert (np.diff(p["worker_offsets"]) >= 0).all()
    loads = np.zeros(W, dtype=np.int64)
    for w in range(W):
        for b, g, i, _ in items[p["worker_offsets"][w]:p["worker_offsets"][w + 1]]:
            loads[w] += min(seq_lens[b], (i + 1) * T) - i * T
    assert np.array_equal(loads, p["loads"])
    assert loads.sum() == Hkv * sum(int(x) for x in seq_lens)
    assert loads.max() - loads.min() <= T


def test_hand_worked_plan():
    with open(os.path.join(GOLDEN, "plan_small.json")) as f:
        g = json.load(f)
    p = P.lpt_plan(g["seq_lens"], g["num_kv_heads"], g["tile_tokens"], g["num_workers"])
    assert p["items"].tolist() == g["items"]
    assert p["worker_offsets"].tolist() == g["worker_offsets"]
    assert p["req_tile_base"].tolist() == g["req_tile_base"]


def test_equal_costs_are_round_robin():
    p = P.lpt_plan([64, 128, 32], 3, 32, 5)
    order = []
    # LPT order of equal-cost items is (b, g, i) ascending; item k goes to worker k mod W
    keys = sorted((b, g, i) for b, L in enumerate([64, 128, 32]) for g in range(3) for i in range(L // 32))
    for k, key in enumerate(keys):
        w = k % 5
        lst = [tuple(x[:3]) for x in p["items"][p["worker_offsets"][w]:p["worker_offsets"][w + 1]]]
        assert key in lst
        order.append(key)
    check_invariants([64, 128, 32], 3, 32, 5, p)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(1, 300), min_size=1, max_size=6), st.integers(1, 3),
       st.sampled_from([16, 32, 48, 64]), st.integers(1, 9))
def test_invariants_random(seq_lens, Hkv, T, W):
    check_invariants(seq_lens, Hkv, T, W, P.lpt_plan(seq_lens, Hkv, T, W))


def brute_force_opt(costs, W):
    best = None
    for assign in itertools.product(range(W), repeat=len(costs)):
        loads = [0] * W
        for c, w in zip(costs, assign):
            loads[w] += c
        m = max(loads)
        best = m if best is None else min(best, m)
    return best


@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(1, 64), min_size=1, max_size=4), st.integers(1, 3))
def test_graham_lpt_bound(seq_lens, W):
    T = 16
    p = P.lpt_plan(seq_lens, 1, T, W)
    costs = [min(L, (i + 1) * T) - i * T for L in seq_lens for i in range((L + T - 1) // T)]
    if len(costs) > 8:
        return
    opt = brute_force_opt(costs, W)
    assert 3 * W * int(p["loads"].max()) <= (4 * W - 1) * opt


def test_fluid_cost_hand_worked():
    # equal loads: one phase of W busy workers -> weight max(W, 160)
    assert P.fluid_cost([5, 5, 5]) == 5 * 160
    assert P.fluid_cost([7] * 200) == 7 * 200
    # 161 workers with 1 token and one with 11 (W = 162): the first token streams with
    # 162 busy workers (1 * 162), the last 10 tokens of the busiest worker alone at the
    # single-worker rate (10 * 160).
    assert P.fluid_cost([1] * 161 + [11]) == 162 + 1600
    # W <= 160: every phase weighs 160, so the cost is 160 * the largest load
    assert P.fluid_cost([3, 9, 1]) == 160 * 9


def test_auto_tile_hand_worked():
    # kv bytes per token = 2*D*eb = 256 (D=64, bf16); item bytes 2^24; partials M*(D+1)*8 = 520.
    # One request of 64 tokens on 4 workers: T=16 -> 4 items, makespan 16:
    # 160*16*256 + 2^24 + 4*520 = 17434656; T=32 -> 160*32*256 + 2^24 + 2*520 = 18088976;
    # T>=64 -> 160*64*256 + 2^24 + 520 = 19399176. So T=16.
    assert P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 4) == 16
    # One worker: T=16 puts 4 items on it (4*2^24); every T >= 64 gives one item and the
    # same estimate, a tie that goes to the largest candidate.
    assert P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 1) == P.MAX_AUTO_TILE
    # One request of 65536 tokens on 64 workers: total/W = 1024 tokens, so the makespan
    # term 160*makespan*256 is minimal (and above the total) at one 1024-token tile per
    # worker; smaller tiles add a second item per worker, larger ones double the makespan.
    assert P.auto_tile_tokens([65536], 1, 1, 1, 64, 16, "bf16", 64) == 1024
    # An item capacity skips the candidates with more items: with at most 3 items T=16
    # (4 items) is out and T=32 (2 items, 18088976) beats T>=64 (19399176); with at most
    # 1 item only T>=64 is left, the tie going to the largest; with 0 none is left.
    assert P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 4, max_items=4) == 16
    assert P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 4, max_items=3) == 32
    assert P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 4, max_items=1) == P.MAX_AUTO_TILE
    with pytest.raises(ValueError):
        P.auto_tile_tokens([64], 1, 1, 1, 64, 16, "bf16", 4, max_items=0)
    # fp8 with page 16: the quantum is lcm(16, 64) = 64
    assert P.tile_quantum(16, "fp8") == 64 and P.tile_quantum(64, "fp8") == 64
    assert P.tile_quantum(32, "bf16") == 32
