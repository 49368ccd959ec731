"""Fused KV append (oracle; test infrastructure only).

The HALOps README (Highlights) lists fused pre/post-processing with its paged-KV
decode attention and an FP8 KV cache, and the HALOps review (sparse attention) has
per-tile FP8 scaling. The step before decode attention writes the step's new tokens
into the paged cache; fused with it here: rotary embedding of the new q and k rows,
and FP8 quantisation of the cache tiles on write. Readings (the pages give none of
these details):

- new tokens: request b's Tq new tokens sit at positions L_b - Tq .. L_b - 1 (L_b
  counts them, as in decode); k_new / v_new are bf16 [B, Tq, Hkv, D]; q is bf16
  [B, Tq, Hq, D];
- rotary embedding (optional): the half-split ("rotate half") form with caller
  tables cos/sin fp32 [max_pos, D/2]: for i < D/2, with c = cos[pos, i],
  s = sin[pos, i], x1 = x[i], x2 = x[i + D/2]:
      x[i]       = fl(fl(x1 * c) - fl(x2 * s))
      x[i + D/2] = fl(fl(x2 * c) + fl(x1 * s))
  every fl() one IEEE float32 rounding (no fused multiply-add); applied to q (all
  heads) and to k, not to v; rotated values are stored rounded to bf16 (nearest even);
- bf16 cache: the (rotated) rows are stored; without rotation they are copied bit
  for bit;
- fp8 cache (OCP e4m3fn, one fp32 scale per page and kv head, K and V separately):
  per page touched, with a = the largest |value| among the new rows of that page:
    * no earlier token in the page (the new rows start at its offset 0):
      scale = fl(a / 448), or 1 if a == 0;
    * else, with the page's current scale s: if fl(a / s) <= 448 the scale stays;
      otherwise scale = fl(a / 448) and every earlier row of the page is re-encoded:
      code' = enc(fl(fl(decode(code) * s) / scale));
    * new rows: code = enc(fl(x / scale));
  enc() rounds to the nearest e4m3fn value (ties to the even code), saturates at
  +-448 and keeps the sign (a negative value that rounds to zero is 0x80).
"""

import numpy as np

from .formats import E4M3FN_TABLE, bf16_bits_to_f64

E4M3_MAX = np.float32(448.0)
# The non-negative finite e4m3fn values and their codes, ascending (codes 0x00-0x7E).
_GRID = E4M3FN_TABLE[:0x7F].astype(np.float64)


def encode_e4m3fn(x):
    """e4m3fn codes (uint8) of float32 values: nearest grid value, ties to the even
    code, saturating at 448, sign kept. NaN maps to 0x7F with its sign."""
    x = np.asarray(x, dtype=np.float32)
    ax = np.abs(x).astype(np.float64)
    hi = np.clip(np.searchsorted(_GRID, ax, side="left"), 0, len(_GRID) - 1)  # first >= ax
    lo = np.maximum(hi - 1, 0)
    d_hi = _GRID[hi] - ax
    d_lo = ax - _GRID[lo]
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(ax >= _GRID[-1], 0x7E, np.where(take_lo, lo, hi)).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code | (np.signbit(x).astype(np.uint8) << 7)


def f32_to_bf16_bits_rne(x):
    """bfloat16 bits of float32 values, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def rope_half(x, c, s):
    """Rotate float32 rows x [..., D] by the tables c, s [..., D/2] (see above)."""
    x = np.asarray(x, dtype=np.float32)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    c = np.asarray(c, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    r1 = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)
    r2 = (x2 * c).astype(np.float32) + (x1 * s).astype(np.float32)
    return np.concatenate([r1.astype(np.float32), r2.astype(np.float32)], axis=-1)


def _append_fp8_page(codes, scales, phys, g, offs, rows):
    """Write float32 rows at offsets offs (ascending, contiguous) of page phys, kv head
    g of an fp8 cache, updating its scale (rule above)."""
    a = np.float32(np.max(np.abs(rows))) if rows.size else np.float32(0)
    o = int(offs[0])
    if o == 0:
        scale = np.float32(a / E4M3_MAX) if a > 0 else np.float32(1.0)
    else:
        s_old = np.float32(scales[phys, g])
        if np.float32(a / s_old) <= E4M3_MAX:
            scale = s_old
        else:
            scale = np.float32(a / E4M3_MAX)
            old = E4M3FN_TABLE[codes[phys, g, :o]].astype(np.float32)
            deq = (old * s_old).astype(np.float32)
            codes[phys, g, :o] = encode_e4m3fn((deq / scale).astype(np.float32))
    scales[phys, g] = scale
    codes[phys, g, offs] = encode_e4m3fn((rows / scale).astype(np.float32))


def kv_append(k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, k_new, v_new, q=None,
              cos=None, sin=None, kv_format="bf16"):
    """Append the step's new tokens in place. Caches, scales: numpy arrays as in the
    decode inputs (uint16 bf16 bits or uint8 codes; fp32 scales); k_new, v_new, q:
    uint16 bf16 bits [B, Tq, H, D]. Returns the rotated q (bf16 bits) when q is given
    with tables, else None."""
    B, Tq, Hkv, D = k_new.shape
    P = k_cache.shape[2]
    rope = cos is not None
    q_out = None
    if rope and q is not None:
        q_out = np.empty_like(q)
    for b in range(B):
        L = int(seq_lens[b])
        pos = np.arange(L - Tq, L)
        if q_out is not None:
            qf = bf16_bits_to_f64(q[b]).astype(np.float32)                  # [Tq, Hq, D]
            q_out[b] = f32_to_bf16_bits_rne(rope_half(qf, cos[pos][:, None], sin[pos][:, None]))
        for g in range(Hkv):
            kf = bf16_bits_to_f64(k_new[b, :, g]).astype(np.float32)        # [Tq, D]
            vf = bf16_bits_to_f64(v_new[b, :, g]).astype(np.float32)
            if rope:
                kf = rope_half(kf, cos[pos], sin[pos])
            for lp in range((L - Tq) // P, (L - 1) // P + 1):
                sel = (pos // P) == lp
                offs = pos[sel] % P
                phys = int(block_table[b, lp])
                if kv_format == "bf16":
                    k_cache[phys, g, offs] = (f32_to_bf16_bits_rne(kf[sel]) if rope
                                              else k_new[b, sel, g])
                    v_cache[phys, g, offs] = v_new[b, sel, g]
                else:
                    _append_fp8_page(k_cache, k_scale, phys, g, offs, kf[sel])
                    _append_fp8_page(v_cache, v_scale, phys, g, offs, vf[sel])
    return q_out
