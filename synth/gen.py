"""Seeded synthetic inputs for paged-KV GQA decode.

This module only draws and encodes random numbers; it holds none of the attention,
softmax, combine or planning arithmetic, and it is the only code that both the HIP
path (tests, bench) and the CPU oracle take inputs from.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):

1. ``seq_lens``: fixed lists as given; ``loguniform``: ``floor(exp(U(ln lo, ln hi)))``
   clipped to [lo, hi]; ``uniform_int``: ``rng.integers(lo, hi + 1)``.
2. Page permutation: ``rng.permutation(num_pages + slack_pages)``. Logical page p of
   request b, taken in (b, p) order, gets the next permutation entry as its physical
   page. Unused block-table entries are -1; ``slack_pages`` pages are never referenced.
3. Q: standard normal float32, rounded to bf16 (round-to-nearest-even on the bits).
4. K pool then V pool, ``[num_pages, Hkv, P, D]``: standard normal float32 drawn in
   chunks of whole pages (same stream as one draw). bf16: rounded as Q. fp8: each
   (page, kv head) tile is scaled by amax/448 (1 if amax is 0) and encoded to OCP
   e4m3fn with round-to-nearest-even, saturating at +-448; the fp32 scale is stored
   in ``k_scale`` / ``v_scale`` ``[num_pages, Hkv]``.

With ``poison=True`` every element no valid token uses (the tail of each request's
last page, and every slack page) is overwritten with NaN bits (bf16 0x7FC0, fp8 0x7F).
Poisoning happens after all draws, so valid data is identical with or without it.
"""

from dataclasses import dataclass
import math

import numpy as np

from .configs import softmax_scale

BF16_NAN = 0x7FC0
FP8_NAN = 0x7F
E4M3_MAX = 448.0

_CHUNK_ELEMS = 1 << 26  # elements per draw chunk (rounded down to whole pages)


@dataclass
class DecodeInputs:
    seq_lens: np.ndarray      # int32 [B]
    block_table: np.ndarray   # int32 [B, max_pages], -1 padding
    q: np.ndarray             # uint16 bf16 bits [B, Tq, Hq, D]
    k_cache: np.ndarray       # uint16 bf16 bits or uint8 e4m3fn codes [num_pages, Hkv, P, D]
    v_cache: np.ndarray
    k_scale: np.ndarray       # float32 [num_pages, Hkv] (fp8) or None
    v_scale: np.ndarray
    scale: float              # fp32-representable softmax scale
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    kv_format: str            # "bf16" | "fp8"

    @property
    def batch(self):
        return int(self.seq_lens.shape[0])

    @property
    def num_pages(self):
        return int(self.k_cache.shape[0])


def f32_to_bf16_bits(x):
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> np.uint32(16)).astype(np.uint16)


def _e4m3fn_grid():
    """The 127 non-negative finite e4m3fn magnitudes, index = code (0x00..0x7E)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_GRID = _e4m3fn_grid()


def f32_to_e4m3fn(x):
    """Encode float values to OCP e4m3fn codes: nearest representable magnitude, ties
    to the even code, saturating to +-448. Inputs are finite; they are taken as
    float32, in which every step below is exact.

    Within a binade [2^e, 2^(e+1)) (e >= -6) the spacing is 2^(e-3); below 2^-6 it is
    2^-9. Rounding mag / spacing to the nearest integer (ties to even) and reading the
    code back from the rounded value gives the code; a rounding up to 2^(e+1) lands on
    the next binade's first code."""
    x = np.asarray(x, dtype=np.float32)
    mag = np.minimum(np.abs(x), np.float32(E4M3_MAX))
    _, ex = np.frexp(mag)                         # mag = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)                    # binade exponent (subnormals share -6)
    step = np.ldexp(np.float32(1.0), e - 3).astype(np.float32)
    q = np.rint(mag / step) * step               # round half to even
    _, qx = np.frexp(q)
    qe = qx - 1
    normal = q >= np.float32(2.0 ** -6)
    m = np.where(normal, np.ldexp(q, -np.maximum(qe, -6)) * 8 - 8, q * 512)
    code = np.where(normal, ((qe + 7) << 3) + m, m).astype(np.uint8)
    sign = (np.signbit(x) & (code != 0)).astype(np.uint8) << 7
    return code | sign


def draw_seq_lens(cfg, rng):
    spec = cfg["seq_lens"]
    B = cfg["batch"]
    if spec[0] == "const":
        return np.full(B, spec[1], dtype=np.int32)
    if spec[0] == "loguniform":
        lo, hi = spec[1], spec[2]
        v = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), B)))
        return np.clip(v, lo, hi).astype(np.int32)
    if spec[0] == "uniform_int":
        return rng.integers(spec[1], spec[2] + 1, B).astype(np.int32)
    return np.asarray(spec, dtype=np.int32)


def _draw_pool(rng, num_pages, Hkv, P, D, kv_format):
    """Draw one K or V pool page-chunk by page-chunk."""
    page_elems = Hkv * P * D
    pages_per_chunk = max(1, _CHUNK_ELEMS // page_elems)
    if kv_format == "bf16":
        pool = np.empty((num_pages, Hkv, P, D), dtype=np.uint16)
        scales = None
    else:
        pool = np.empty((num_pages, Hkv, P, D), dtype=np.uint8)
        scales = np.empty((num_pages, Hkv), dtype=np.float32)
    for p0 in range(0, num_pages, pages_per_chunk):
        n = min(pages_per_chunk, num_pages - p0)
        x = rng.standard_normal(n * page_elems, dtype=np.float32).reshape(n, Hkv, P, D)
        if kv_format == "bf16":
            pool[p0:p0 + n] = f32_to_bf16_bits(x)
        else:
            amax = np.abs(x).max(axis=(2, 3))
            s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
            scales[p0:p0 + n] = s
            pool[p0:p0 + n] = f32_to_e4m3fn(x / s[:, :, None, None])
    return pool, scales


def make_inputs(cfg, seed=0, poison=False, slack_pages=0, seq_lens=None):
    """Draw a full decode batch for workload ``cfg`` (see the module recipe).

    ``seq_lens`` overrides the workload's lengths (used by edge-case tests)."""
    rng = np.random.default_rng(seed)
    B, Tq = cfg["batch"], cfg["q_len"]
    Hq, Hkv, D, P = cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["page_size"]
    fmt = cfg["kv_format"]
    if seq_lens is None:
        seq_lens = draw_seq_lens(cfg, rng)
    else:
        seq_lens = np.asarray(seq_lens, dtype=np.int32)
        B = int(seq_lens.shape[0])
    pages = [(int(L) + P - 1) // P for L in seq_lens]
    num_used = int(sum(pages))
    num_pages = num_used + int(slack_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    max_pages = max(pages) if pages else 1
    block_table = np.full((B, max(max_pages, 1)), -1, dtype=np.int32)
    k = 0
    for b in range(B):
        block_table[b, :pages[b]] = perm[k:k + pages[b]]
        k += pages[b]
    q = f32_to_bf16_bits(rng.standard_normal(B * Tq * Hq * D, dtype=np.float32)).reshape(B, Tq, Hq, D)
    k_cache, k_scale = _draw_pool(rng, num_pages, Hkv, P, D, fmt)
    v_cache, v_scale = _draw_pool(rng, num_pages, Hkv, P, D, fmt)
    inp = DecodeInputs(seq_lens=seq_lens, block_table=block_table, q=q,
                       k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
                       scale=float(np.float32(softmax_scale(D))), q_len=Tq,
                       num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                       kv_format=fmt)
    if poison:
        apply_poison(inp)
    return inp


@dataclass
class PrefillInputs:
    cache: DecodeInputs       # seq_lens = kv lengths (prefix + query tokens), block table, pools
    q: np.ndarray             # uint16 bf16 bits [total_q, Hq, D], requests packed in order
    q_lens: np.ndarray        # int32 [B]
    cu_q: np.ndarray          # int32 [B + 1], prefix sums of q_lens

    @property
    def batch(self):
        return int(self.q_lens.shape[0])


def make_prefill_inputs(cfg, seed=0, q_lens=None, prefix=None, poison=False, slack_pages=0):
    """Draw a prefill batch: q lengths then prefixes from ``default_rng(seed)`` (recipes
    as for seq_lens), the cache of kv lengths prefix + q length from ``make_inputs``
    with seed + 1, then the packed q (standard normal, bf16) from ``default_rng(seed +
    2)``. ``q_lens`` / ``prefix`` override the recipes."""
    rng = np.random.default_rng(seed)
    B = cfg["batch"]
    if q_lens is None:
        q_lens = draw_seq_lens(dict(batch=B, seq_lens=cfg["q_lens"]), rng)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    B = int(q_lens.shape[0])
    if prefix is None:
        prefix = draw_seq_lens(dict(batch=B, seq_lens=cfg["prefix"]), rng)
    prefix = np.asarray(prefix, dtype=np.int32)
    kv = (q_lens + prefix).astype(np.int32)
    cache_cfg = dict(cfg, q_len=1, seq_lens=tuple(int(x) for x in kv), batch=B)
    cache = make_inputs(cache_cfg, seed=seed + 1, poison=poison, slack_pages=slack_pages)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    total = int(cu[-1])
    rq = np.random.default_rng(seed + 2)
    H, D = cfg["num_q_heads"], cfg["head_dim"]
    q = f32_to_bf16_bits(rq.standard_normal(total * H * D, dtype=np.float32)).reshape(total, H, D)
    return PrefillInputs(cache=cache, q=q, q_lens=q_lens, cu_q=cu)


def prefill_flops(inp):
    """Algorithmic flops of causal prefill attention: 4 * D * Hq per (query, visible
    key) pair (Q.K and P.V, multiply-add = 2), query t of request b seeing
    prefix_b + t + 1 keys."""
    c = inp.cache
    pairs = 0
    for b in range(inp.batch):
        n = int(inp.q_lens[b])
        pre = int(c.seq_lens[b]) - n
        pairs += n * pre + n * (n + 1) // 2
    return 4 * c.head_dim * c.num_q_heads * pairs


def apply_poison(inp):
    """Overwrite every element that no valid token reads with NaN bits."""
    nan = BF16_NAN if inp.kv_format == "bf16" else FP8_NAN
    P = inp.page_size
    used = np.zeros(inp.num_pages, dtype=bool)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        n = (L + P - 1) // P
        used[inp.block_table[b, :n]] = True
        tail = L - (n - 1) * P
        if tail < P:
            last = inp.block_table[b, n - 1]
            inp.k_cache[last, :, tail:, :] = nan
            inp.v_cache[last, :, tail:, :] = nan
    inp.k_cache[~used] = nan
    inp.v_cache[~used] = nan
    return inp


def rope_tables(max_pos, head_dim, base=10000.0):
    """Rotary-embedding tables: cos and sin of pos * base^(-2i/D), i < D/2, computed
    in float64 and stored as float32 [max_pos, D/2] (inputs of the append)."""
    inv = base ** (-np.arange(head_dim // 2, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def new_token_rows(inp, seed=0, scale=1.0):
    """The step's new k and v rows (bf16 bits [B, Tq, Hkv, D]) and a new q (bf16 bits
    [B, Tq, Hq, D]), standard normal times ``scale`` (a scalar or a [B, Hkv] array)."""
    rng = np.random.default_rng(seed)
    B, Tq, Hkv, D = inp.batch, inp.q_len, inp.num_kv_heads, inp.head_dim
    sc = np.broadcast_to(np.asarray(scale, np.float32), (B, Hkv))[:, None, :, None]
    k = f32_to_bf16_bits((rng.standard_normal((B, Tq, Hkv, D), dtype=np.float32) * sc).astype(np.float32))
    v = f32_to_bf16_bits((rng.standard_normal((B, Tq, Hkv, D), dtype=np.float32) * sc).astype(np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((B, Tq, inp.num_q_heads, D), dtype=np.float32))
    return k, v, q


def append_algorithmic_bytes(inp, rope=True):
    """Bytes the fused append must move at minimum: the new k and v rows read (bf16)
    and written to the cache, q read and written rotated, the rotation table rows of
    the new positions, the block-table entries of the touched pages, seq_lens and
    (fp8) the touched pages' scales read and written."""
    eb = 2 if inp.kv_format == "bf16" else 1
    B, Tq, Hkv, Hq, D, P = (inp.batch, inp.q_len, inp.num_kv_heads, inp.num_q_heads,
                            inp.head_dim, inp.page_size)
    rows = B * Tq * Hkv * D
    touched = sum((int(L) - 1) // P - (int(L) - Tq) // P + 1 for L in inp.seq_lens)
    total = 2 * rows * 2 + 2 * rows * eb + 4 * touched + 4 * B
    if rope:
        total += 2 * B * Tq * Hq * D * 2 + 2 * B * Tq * (D // 2) * 4
    if inp.kv_format != "bf16":
        total += 2 * 2 * 4 * touched * Hkv
    return total


def make_block_mask(inp, keep, seed=1):
    """Block mask for block-sparse decode: uint8 [B, Hkv, bt_stride], 1 = page
    attended, each (request, kv head, logical page) kept with probability ``keep``
    (its own generator, so the inputs of ``make_inputs`` are unchanged)."""
    rng = np.random.default_rng(seed)
    shape = (inp.batch, inp.num_kv_heads, inp.block_table.shape[1])
    return (rng.random(shape) < keep).astype(np.uint8)


def attended_pages(inp, block_mask):
    """Per (request, kv head): the logical pages block-sparse decode reads - the
    masked-in pages plus those holding the step's query tokens. List of lists."""
    P, Tq = inp.page_size, inp.q_len
    out = []
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        n = (L + P - 1) // P
        first_query_page = (L - Tq) // P
        out.append([[p for p in range(n) if block_mask[b, g, p] or p >= first_query_page]
                    for g in range(inp.num_kv_heads)])
    return out


def sparse_algorithmic_bytes(inp, block_mask, decode_only=False):
    """Bytes a block-sparse decode step must move at minimum: K and V of the
    attended tokens, Q, the bf16 output, the mask entries and block-table entries of
    every page, seq_lens and (fp8) the scales of attended pages. ``decode_only``: the
    share of the split-KV partial kernel - attended K/V, Q, one compacted block-table
    entry per attended page, the compacted lengths and the attended pages' scales."""
    eb = 2 if inp.kv_format == "bf16" else 1
    P = inp.page_size
    tokens = pages_att = pages_all = 0
    for b, per_g in enumerate(attended_pages(inp, block_mask)):
        L = int(inp.seq_lens[b])
        n = (L + P - 1) // P
        pages_all += n
        for pages in per_g:
            pages_att += len(pages)
            tokens += sum(min(P, L - p * P) for p in pages)
    kv = tokens * inp.head_dim * eb * 2
    q = inp.batch * inp.q_len * inp.num_q_heads * inp.head_dim * 2
    scales = 0 if inp.kv_format == "bf16" else 2 * 4 * pages_att
    if decode_only:
        return kv + q + 4 * pages_att + 4 * inp.batch * inp.num_kv_heads + scales
    return kv + 2 * q + 4 * pages_all + pages_all * inp.num_kv_heads + 4 * inp.batch + scales


def algorithmic_bytes(inp):
    """Bytes the decode step must move at minimum: K and V of every valid token,
    Q, the bf16 output, the block-table entries used, seq_lens and (fp8) the scales
    of the pages used. Split-KV partials are excluded."""
    eb = 2 if inp.kv_format == "bf16" else 1
    P = inp.page_size
    sl = inp.seq_lens.astype(np.int64)
    pages = (sl + P - 1) // P
    kv = int(sl.sum()) * inp.num_kv_heads * inp.head_dim * eb * 2
    q = inp.batch * inp.q_len * inp.num_q_heads * inp.head_dim * 2
    bt = 4 * int(pages.sum())
    scales = 0 if inp.kv_format == "bf16" else 2 * 4 * int(pages.sum()) * inp.num_kv_heads
    return kv + 2 * q + bt + 4 * inp.batch + scales
