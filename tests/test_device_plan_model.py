"""CPU model of the device planner's steps against the oracle's one-at-a-time LPT.

The device planner (the HIP kernel behind pkv_plan_device) does not run the oracle's
heap. It places the full tiles round-robin in closed form, then the remainder tiles in
batches: with the worker keys (load relative to a reference, worker index) sorted
ascending, item k + j goes to the j-th key while that key is below every key already
raised in the batch, and the keys are sorted again after each batch. Its streaming term
is the summation-by-parts form of the oracle's fluid cost. This file restates those
steps in plain Python, with the kernel's 32-bit key packing, and checks on random
batches that they give the oracle's plan item for item and the oracle's estimate. It
pins the argument the kernel rests on; the kernel itself is compared with the oracle on
the GPU.
"""

import numpy as np
import pytest

from oracle import plan as oracle_plan

WORKER_BITS = 10  # worker index in the low bits of a worker key
REQ_BITS = 13     # request index in the low bits of a remainder key


def device_model(seq_lens, Hkv, T, W):
    """(items [N, 4], worker_offsets [W + 1], loads [W] by worker, number of batches,
    loads sorted ascending)."""
    L = np.asarray(seq_lens, dtype=np.int64)
    B = len(L)
    f = L // T
    c = L - f * T
    n = f + (c != 0)
    rtb = np.concatenate([[0], np.cumsum(n)])
    fbx = np.concatenate([[0], np.cumsum(f)])[:-1] * Hkv   # first full item of request b
    F = int(f.sum()) * Hkv
    base, r = divmod(F, W)
    ref = base * T
    # Sorted worker keys after the round-robin: workers r .. W-1 at `ref`, 0 .. r-1 one
    # tile above.
    keys = [((T if w < r else 0) << WORKER_BITS) | w for w in list(range(r, W)) + list(range(r))]
    # Remainder items: requests by (T - c) << REQ_BITS | b ascending, each Hkv times.
    rkeys = sorted(((T - int(c[b])) << REQ_BITS) | b for b in range(B) if c[b] != 0)
    items_c = [(rk & ((1 << REQ_BITS) - 1), g) for rk in rkeys for g in range(Hkv)]
    K = len(items_c)
    assign = [None] * K
    wcnt = [0] * W
    k = batches = 0
    while k < K:
        lim = min(W, K - k)
        raised = []
        np_ = lim
        below = None
        for j in range(lim):
            if below is not None and keys[j] > below:
                np_ = j
                break
            cost = int(c[items_c[k + j][0]])
            rj = keys[j] + (cost << WORKER_BITS)
            raised.append(rj)
            below = rj if below is None else min(below, rj)
        for j in range(np_):
            w = keys[j] & ((1 << WORKER_BITS) - 1)
            assign[k + j] = (w, wcnt[w])
            wcnt[w] += 1
            keys[j] = raised[j]
        keys.sort()
        d = keys[0] >> WORKER_BITS      # re-base on the least load
        keys = [key - (d << WORKER_BITS) for key in keys]
        ref += d
        assert all(key < (1 << 31) for key in keys), "32-bit worker keys"
        k += np_
        batches += 1
    loads_sorted = [ref + (key >> WORKER_BITS) for key in keys]
    worker_of_key = [key & ((1 << WORKER_BITS) - 1) for key in keys]
    loads = np.zeros(W, dtype=np.int64)
    for w, l in zip(worker_of_key, loads_sorted):
        loads[w] = l
    counts = [base + (1 if w < r else 0) + wcnt[w] for w in range(W)]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    items = np.zeros((int(offsets[-1]), 4), dtype=np.int64)
    # Full items: the x-th in (b, g, i) order goes to worker x mod W at position x / W,
    # written per (request, kv head) pair as the kernel does.
    for b in range(B):
        for g in range(Hkv):
            x0 = int(fbx[b]) + g * int(f[b])
            for i in range(int(f[b])):
                x = x0 + i
                items[offsets[x % W] + x // W] = (b, g, i, Hkv * rtb[b] + g * n[b] + i)
    for x, (b, g) in enumerate(items_c):
        w, pos = assign[x]
        fw = base + (1 if w < r else 0)
        i = int(f[b])
        items[offsets[w] + fw + pos] = (b, g, i, Hkv * rtb[b] + g * n[b] + i)
    return items, offsets, loads, batches, sorted(loads_sorted)


def fluid_by_parts(sorted_loads):
    """The kernel's form: the W - R smallest loads plus R times the largest (R = the
    worker ratio), or R times the largest when W <= R."""
    R = oracle_plan.WORKER_RATIO
    W = len(sorted_loads)
    if W <= R:
        return R * sorted_loads[-1]
    return sum(sorted_loads[:W - R]) + R * sorted_loads[-1]


def random_case(rng):
    B = int(rng.integers(1, 40))
    T = int(rng.choice([16, 48, 64, 256, 1024, 4096]))
    mode = rng.integers(3)
    if mode == 0:
        L = rng.integers(1, 6 * T, B)
    elif mode == 1:
        L = np.exp(rng.uniform(0, np.log(20 * T), B)).astype(np.int64) + 1
    else:
        L = T * rng.integers(0, 4, B) + rng.integers(1, 3, B)   # near tile multiples
    Hkv = int(rng.choice([1, 2, 3, 8]))
    W = int(rng.choice([1, 3, 7, 100, 161, 256, 300]))
    return [int(x) for x in L], Hkv, T, W


@pytest.mark.parametrize("seed", range(6))
def test_device_steps_give_the_oracle_plan(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        sl, Hkv, T, W = random_case(rng)
        ref = oracle_plan.lpt_plan(sl, Hkv, T, W)
        items, offsets, loads, _, _ = device_model(sl, Hkv, T, W)
        assert np.array_equal(offsets, ref["worker_offsets"]), (sl, Hkv, T, W)
        assert np.array_equal(items, ref["items"]), (sl, Hkv, T, W)
        assert np.array_equal(loads, ref["loads"]), (sl, Hkv, T, W)


@pytest.mark.parametrize("seed", range(4))
def test_summation_by_parts_equals_the_fluid_cost(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(60):
        sl, Hkv, T, W = random_case(rng)
        _, _, loads, _, sorted_loads = device_model(sl, Hkv, T, W)
        assert fluid_by_parts(sorted_loads) == oracle_plan.fluid_cost(loads)


def test_mixed_batches_are_few_and_large():
    """The mixed-length workload's remainder tiles go in a handful of batches at the
    default 256 workers (the kernel's cost is per batch)."""
    import synth
    cfg = synth.ALL["mixed"]
    sl = synth.gen.draw_seq_lens(cfg, np.random.default_rng(0))
    for T in (4096, 16384, 65536):
        items, offsets, loads, batches, _ = device_model(sl, cfg["num_kv_heads"], T, 256)
        ref = oracle_plan.lpt_plan(sl, cfg["num_kv_heads"], T, 256)
        assert np.array_equal(items, ref["items"])
        assert batches <= 6


def wave_exclusive_min(values):
    """The kernel's in-wave butterfly: at level j each lane takes its partner block's
    minimum (lane ^ j), which joins the lane's prefix when that block lies below it."""
    total = list(values)
    excl = [0xFFFFFFFF] * 64
    j = 1
    while j < 64:
        other = [total[lane ^ j] for lane in range(64)]
        excl = [min(e, o) if lane & j else e for lane, (e, o) in enumerate(zip(excl, other))]
        total = [min(t, o) for t, o in zip(total, other)]
        j *= 2
    return excl, total


def test_wave_butterfly_is_the_exclusive_prefix_minimum():
    rng = np.random.default_rng(7)
    for _ in range(500):
        v = [int(x) for x in rng.integers(0, 1 << 31, 64)]
        for lane in rng.integers(0, 64, int(rng.integers(0, 20))):
            v[lane] = 0xFFFFFFFF          # lanes past the batch hold the sentinel
        excl, total = wave_exclusive_min(v)
        assert excl == [min(v[:lane], default=0xFFFFFFFF) for lane in range(64)]
        assert total == [min(v)] * 64
