"""Reference tile planner: uniform KV tiles + greedy (LPT) bin-packing onto workers.

The HPC-Ops review ("How the kernels are organized around specific workload
shapes", and the FlashInfer comparison section's "task map" for mixed-length
decode) describes the scheduler: before every decode step each request's KV is cut
into tiles of one uniform size and the tiles are spread over the thread blocks by
greedy bin-packing, because a fixed split count cannot balance a batch whose KV
lengths differ. The pages give no cost, order or tie rule; the readings here:

- work item (b, g, i): kv head g of request b, tokens [i*T, min(L_b, (i+1)*T)),
  i < n_b = ceil(L_b / T); its cost is its token count;
- greedy = longest-processing-time first: items sorted by cost descending, ties by
  (b, g, i) ascending; each goes to the worker with the least load so far, ties to
  the lowest worker index; a worker's items are kept in assignment order;
- partial slot of item (b, g, i): Hkv * req_tile_base[b] + g * n_b + i, where
  req_tile_base is the prefix sum of n_b;
- automatic tile size (tile_tokens == 0), a bandwidth-sharing cost model:
  candidates quantum * 2**k <= 65536 (quantum = page size for bf16,
  lcm(page size, 64) for fp8); the estimate
      kv * fluid(worker loads) + max_items_per_worker * ITEM_BYTES + N * M * (D + 1) * 8
  (kv = 2 * D * eb bytes per token) is minimised, ties going to the larger tile.
  fluid() is the streaming time of the plan on a memory-bound chip, in chip-byte
  units: while k workers are busy each streams at min(chip / k, chip / WORKER_RATIO),
  so with the loads sorted ascending, l_1 <= ... <= l_W (l_0 = 0),
      fluid = sum_j (l_j - l_(j-1)) * max(W - j + 1, WORKER_RATIO).
  It equals the total when enough workers stay busy to the end and grows with the
  tail the busiest workers leave. WORKER_RATIO (how many workers saturate the chip)
  and ITEM_BYTES (the fixed cost of one work item in chip-wide bytes, ~2.6 us at
  ~6.5 TB/s) come from measurements on MI355X and are kept as a pair: together they
  pick the fastest measured power-of-two tile on every benchmark workload, although
  one eight-wave workgroup alone streams at about chip / 240 rather than chip / 160.
  The last term is the partials written and read back by the combine.

This is the plain definition (a full sort and a heap over every item); the native
planner uses an equivalent faster form and must match it bit for bit.
"""

import heapq
import math

import numpy as np

MAX_AUTO_TILE = 65536
WORKER_RATIO = 160
ITEM_BYTES = 1 << 24


def fluid_cost(loads):
    """Streaming time of per-worker token loads in chip-token units (see above)."""
    l = sorted(int(x) for x in loads)
    W = len(l)
    total, prev = 0, 0
    for j, x in enumerate(l):
        total += (x - prev) * max(W - j, WORKER_RATIO)
        prev = x
    return total


def num_tiles(L, T):
    return (int(L) + T - 1) // T


def tile_quantum(page_size, kv_format):
    if kv_format == "bf16":
        return page_size
    return page_size * 64 // math.gcd(page_size, 64)


def lpt_plan(seq_lens, num_kv_heads, T, W):
    """Return dict(items [N,4] int32 rows (b, g, i, slot), worker_offsets [W+1],
    req_tile_base [B+1], loads [W] int64, tile_tokens T)."""
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    nb = [num_tiles(L, T) for L in seq_lens]
    rtb = np.zeros(B + 1, dtype=np.int64)
    rtb[1:] = np.cumsum(nb)
    items = []
    for b in range(B):
        for g in range(num_kv_heads):
            for i in range(nb[b]):
                cost = min(seq_lens[b], (i + 1) * T) - i * T
                slot = num_kv_heads * int(rtb[b]) + g * nb[b] + i
                items.append((cost, b, g, i, slot))
    items.sort(key=lambda it: (-it[0], it[1], it[2], it[3]))
    heap = [(0, w) for w in range(W)]
    lists = [[] for _ in range(W)]
    loads = np.zeros(W, dtype=np.int64)
    for cost, b, g, i, slot in items:
        load, w = heapq.heappop(heap)
        lists[w].append((b, g, i, slot))
        loads[w] = load + cost
        heapq.heappush(heap, (load + cost, w))
    offsets = np.zeros(W + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(x) for x in lists])
    flat = [it for lst in lists for it in lst]
    arr = np.array(flat, dtype=np.int32).reshape(-1, 4)
    return dict(items=arr, worker_offsets=offsets, req_tile_base=rtb.astype(np.int32),
                loads=loads, tile_tokens=T)


def auto_tile_tokens(seq_lens, q_len, num_q_heads, num_kv_heads, head_dim, page_size,
                     kv_format, W, max_items=None):
    """The automatic tile size (see module docstring). With ``max_items`` (the item
    capacity of a plan built on the device) candidates whose plan has more items are
    skipped; ValueError if none is left."""
    quantum = tile_quantum(page_size, kv_format)
    eb = 2 if kv_format == "bf16" else 1
    M = (num_q_heads // num_kv_heads) * q_len
    cands = []
    T = quantum
    while True:
        cands.append(T)
        if T * 2 > MAX_AUTO_TILE:
            break
        T *= 2
    best_T, best_est = None, None
    for T in cands:
        p = lpt_plan(seq_lens, num_kv_heads, T, W)
        counts = np.diff(p["worker_offsets"]).astype(np.int64)
        N = int(counts.sum())
        if max_items is not None and N > max_items:
            continue
        kv = 2 * head_dim * eb
        est = kv * fluid_cost(p["loads"]) + int(counts.max()) * ITEM_BYTES + N * M * (head_dim + 1) * 8
        if best_est is None or est < best_est or (est == best_est and T > best_T):
            best_T, best_est = T, est
    if best_T is None:
        raise ValueError("no candidate tile has at most %d items" % max_items)
    return best_T


def plan(seq_lens, q_len, num_q_heads, num_kv_heads, head_dim, page_size, kv_format,
         tile_tokens, W, max_items=None):
    """Resolve the tile size (0 = automatic) and build the plan."""
    T = tile_tokens or auto_tile_tokens(seq_lens, q_len, num_q_heads, num_kv_heads,
                                        head_dim, page_size, kv_format, W, max_items)
    return lpt_plan(seq_lens, num_kv_heads, T, W)
