"""Plain fp64 paged-KV GQA decode attention (oracle; test infrastructure only).

What is computed. The HALOps README (Highlights) lists decode attention over a
paged KV cache with grouped-query heads, BF16 or FP8 KV and speculative decoding;
the HPC-Ops review ("How the kernels are organized around specific workload
shapes") says split-KV partial results are merged by a combine kernel. Split-KV plus
an exact merge can only reproduce ordinary softmax attention, so this module writes
that definition out directly, with no tiling and no online softmax:

For request b, query token t < Tq, query head h (kv head g = h // G, G = Hq/Hkv):
  pos   = L_b - Tq + t                      (the draft token's own position)
  K_b[j] = dequant(k_cache[block_table[b, j // P], g, j % P, :])   for j < L_b
  s_j   = scale * <q[b,t,h], K_b[j]>        for j <= pos  (causal inside the draft)
  p_j   = exp(s_j - max s) / sum_{j'<=pos} exp(s_j' - max s)
  out   = sum_j p_j V_b[j]
  lse   = max s + ln sum_j exp(s_j - max s)

Readings of points the pages leave open (each also listed in the design notes):
- cache layout [num_pages, Hkv, P, D], D innermost, K and V separate;
- block table int32 [B, stride], entry (b, p) = physical page of logical page p;
- q head h reads kv head h // G;
- seq_lens include the Tq draft tokens; row t sees keys 0 .. L-Tq+t;
- FP8 is OCP e4m3fn; one fp32 scale per (physical page, kv head) for K and for V,
  the dequantised value being code_value * scale.

Everything is evaluated in float64 from the exact stored values (bf16 bits and
e4m3fn codes decode exactly; code * fp32 scale is exact in float64).

Block-sparse decode (the HALOps review's sparse attention: a precomputed block mask,
masked-out KV tiles skipped, per-tile FP8 scaling kept). Readings: one mask entry per
(request, kv head, logical page), nonzero = attended; the pages that hold the step's
own query tokens (positions L-Tq .. L-1) are always attended, so a query always
sees itself. The key set of row t is then
  { j <= pos : block_mask[b, g, j // P] != 0  or  j // P >= (L - Tq) // P }.
"""

import numpy as np

from .formats import bf16_bits_to_f64, e4m3fn_to_f64


def gather_kv(cache, scales, block_table_row, L, g, page_size, kv_format):
    """Dequantised keys (or values) of one request and kv head: float64 [L, D]."""
    n_pages = (L + page_size - 1) // page_size
    phys = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    pages = cache[phys, g]                              # [n_pages, P, D]
    if kv_format == "bf16":
        x = bf16_bits_to_f64(pages)
    else:
        x = e4m3fn_to_f64(pages) * scales[phys, g].astype(np.float64)[:, None, None]
    return x.reshape(n_pages * page_size, -1)[:L]


def sparse_keys(mask_row, L, q_len, pos, page_size):
    """Positions j <= pos attended under one (request, kv head) block-mask row."""
    first_query_page = (L - q_len) // page_size
    return [j for j in range(pos + 1)
            if mask_row[j // page_size] != 0 or j // page_size >= first_query_page]


def decode_attention(inp, pairs=None, block_mask=None):
    """Reference decode attention for a ``synth.DecodeInputs`` batch.

    Returns (out, lse): out float64 [B, Tq, Hq, D], lse float64 [B, Tq, Hq] (natural
    log). With ``pairs`` (an iterable of (b, g)), only those request / kv-head groups
    are computed and every other entry is NaN. ``block_mask`` (uint8 [B, Hkv, >=
    pages]) restricts the keys to the attended pages (block-sparse decode).
    """
    B, Tq = inp.batch, inp.q_len
    Hq, Hkv, D, P = inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size
    G = Hq // Hkv
    out = np.full((B, Tq, Hq, D), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    q = bf16_bits_to_f64(inp.q)
    scale = float(np.float32(inp.scale))
    if pairs is None:
        pairs = [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        L = int(inp.seq_lens[b])
        K = gather_kv(inp.k_cache, inp.k_scale, inp.block_table[b], L, g, P, inp.kv_format)
        V = gather_kv(inp.v_cache, inp.v_scale, inp.block_table[b], L, g, P, inp.kv_format)
        for t in range(Tq):
            pos = L - Tq + t
            if block_mask is None:
                Kt, Vt = K[:pos + 1], V[:pos + 1]
            else:
                idx = sparse_keys(block_mask[b, g], L, Tq, pos, P)
                Kt, Vt = K[idx], V[idx]
            qh = q[b, t, g * G:(g + 1) * G, :]          # [G, D]
            s = scale * (qh @ Kt.T)                     # [G, pos+1]
            mx = s.max(axis=1, keepdims=True)
            e = np.exp(s - mx)
            den = e.sum(axis=1, keepdims=True)
            out[b, t, g * G:(g + 1) * G] = (e / den) @ Vt
            lse[b, t, g * G:(g + 1) * G] = mx[:, 0] + np.log(den[:, 0])
    return out, lse


def attention_probs(q_row, K, scale):
    """Softmax probabilities of one query row over keys K (float64)."""
    s = scale * (K @ q_row)
    e = np.exp(s - s.max())
    return e / e.sum()


def partial_attention(q_rows, K, V, scale, key_idx):
    """Attention of ``q_rows`` [R, D] over the key subset ``key_idx`` only.

    Returns (o [R, D] normalised over the subset, lse [R]). An empty subset gives
    o = 0 and lse = -inf, the identity of the log-sum-exp merge."""
    R, D = q_rows.shape
    if len(key_idx) == 0:
        return np.zeros((R, V.shape[1])), np.full(R, -np.inf)
    s = scale * (q_rows @ K[key_idx].T)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    return (e / den) @ V[key_idx], mx[:, 0] + np.log(den[:, 0])
