"""Variable-length causal prefill attention over the paged cache (oracle; test
infrastructure only).

The HALOps README (Highlights) lists variable-length prefill next to paged-KV decode
for its GQA attention; the HPC-Ops launch article measures prefill for inputs of 128
to 64K tokens. Readings: a batch packs the query rows of B requests (q [total, Hq, D],
request b's rows at cu_q[b] .. cu_q[b+1]-1); request b's q_len_b query tokens are the
last q_len_b of its L_b cached tokens (a whole prompt when L_b == q_len_b, a chunk
after a prefix otherwise), so query t sits at position pos = L_b - q_len_b + t and
attends to the keys j <= pos (causal); q head h reads kv head h // G; the cache, the
block table and FP8 dequantisation are those of decode.

For each row: s_j = scale * <q_t, K[j]> (j <= pos), p = softmax(s), out = p . V,
lse = max s + ln sum exp(s - max s); float64 throughout. Rows are evaluated a chunk
at a time with an explicit mask (each row's arithmetic is the definition above).
"""

import numpy as np

from .attention import gather_kv
from .formats import bf16_bits_to_f64

ROW_CHUNK = 256


def prefill_attention(inp, pairs=None, rows=None):
    """Reference prefill for a ``synth.PrefillInputs`` batch.

    Returns (out float64 [total, Hq, D], lse float64 [total, Hq]). ``pairs`` (iterable
    of (b, g)) limits the work to those request / kv-head groups; ``rows`` (dict
    b -> iterable of query indices t) limits it further to those query tokens.
    Entries not computed are NaN."""
    c = inp.cache
    Hq, Hkv, D, P = c.num_q_heads, c.num_kv_heads, c.head_dim, c.page_size
    G = Hq // Hkv
    total = int(inp.cu_q[-1])
    out = np.full((total, Hq, D), np.nan)
    lse = np.full((total, Hq), np.nan)
    scale = float(np.float32(c.scale))
    if pairs is None:
        pairs = [(b, g) for b in range(inp.batch) for g in range(Hkv)]
    for b, g in pairs:
        L, n, q0 = int(c.seq_lens[b]), int(inp.q_lens[b]), int(inp.cu_q[b])
        K = gather_kv(c.k_cache, c.k_scale, c.block_table[b], L, g, P, c.kv_format)
        V = gather_kv(c.v_cache, c.v_scale, c.block_table[b], L, g, P, c.kv_format)
        ts = np.arange(n) if rows is None or b not in rows else np.asarray(sorted(rows[b]), int)
        for i0 in range(0, len(ts), ROW_CHUNK):
            t = ts[i0:i0 + ROW_CHUNK]
            pos = L - n + t                                        # [R]
            qh = bf16_bits_to_f64(inp.q[q0 + t, g * G:(g + 1) * G, :])   # [R, G, D]
            hi = int(pos.max()) + 1
            s = scale * np.einsum("rgd,jd->rgj", qh, K[:hi])      # [R, G, hi]
            visible = np.arange(hi)[None, :] <= pos[:, None]      # [R, hi]
            s = np.where(visible[:, None, :], s, -np.inf)
            mx = s.max(axis=2, keepdims=True)
            e = np.exp(s - mx)
            den = e.sum(axis=2, keepdims=True)
            out[q0 + t, g * G:(g + 1) * G] = np.einsum("rgj,jd->rgd", e / den, V[:hi])
            lse[q0 + t, g * G:(g + 1) * G] = mx[:, :, 0] + np.log(den[:, :, 0])
    return out, lse
