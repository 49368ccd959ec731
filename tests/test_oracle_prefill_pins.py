"""Pins of the prefill oracle (CPU only), against things other than itself:
- q_len = Tq for every request reduces to the decode oracle;
- torch's float64 scaled_dot_product_attention with an explicit causal-with-offset
  mask on a dense copy of each request's cache (torch's own bf16 / e4m3fn decoders);
- causality: keys after a row's position never change that row;
- chunked prefill: a chunk's rows equal the same rows of a whole-prompt prefill.
"""

import copy

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.prefill import prefill_attention


def cfg(**kw):
    base = dict(name="p", batch=0, q_lens=("const", 1), prefix=("const", 0), num_q_heads=4,
                num_kv_heads=2, head_dim=16, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def test_reduces_to_decode_when_every_request_has_tq_tokens():
    Tq = 3
    p = synth.make_prefill_inputs(cfg(), seed=1, q_lens=[Tq] * 4, prefix=[2, 14, 30, 61])
    out, lse = prefill_attention(p)
    d = copy.deepcopy(p.cache)
    d.q = p.q.reshape(4, Tq, d.num_q_heads, d.head_dim)
    d.q_len = Tq
    ref_out, ref_lse = oracle.decode_attention(d)
    np.testing.assert_allclose(out, ref_out.reshape(out.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.reshape(lse.shape), rtol=0, atol=1e-12)


def torch_reference(p):
    """Dense per-request K/V through the block table, torch decoders, torch SDPA."""
    c = p.cache
    Hq, Hkv, D, P = c.num_q_heads, c.num_kv_heads, c.head_dim, c.page_size
    G = Hq // Hkv
    outs = []
    if c.kv_format == "bf16":
        kd = torch.from_numpy(c.k_cache.view(np.int16).copy()).view(torch.bfloat16).double()
        vd = torch.from_numpy(c.v_cache.view(np.int16).copy()).view(torch.bfloat16).double()
    else:
        ks = torch.from_numpy(c.k_scale.astype(np.float64))[:, :, None, None]
        vs = torch.from_numpy(c.v_scale.astype(np.float64))[:, :, None, None]
        kd = torch.from_numpy(c.k_cache.copy()).view(torch.float8_e4m3fn).double() * ks
        vd = torch.from_numpy(c.v_cache.copy()).view(torch.float8_e4m3fn).double() * vs
    q = torch.from_numpy(p.q.view(np.int16).copy()).view(torch.bfloat16).double()
    for b in range(p.batch):
        L, n, q0 = int(c.seq_lens[b]), int(p.q_lens[b]), int(p.cu_q[b])
        pages = torch.from_numpy(c.block_table[b, :(L + P - 1) // P].astype(np.int64))
        K = kd[pages].permute(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :L].repeat_interleave(G, 0)
        V = vd[pages].permute(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :L].repeat_interleave(G, 0)
        qb = q[q0:q0 + n].permute(1, 0, 2)                       # [Hq, n, D]
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qb, K, V, attn_mask=mask,
                                                             scale=float(np.float32(c.scale)))
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs)


@pytest.mark.parametrize("kw,q_lens,prefix", [
    (dict(), [1, 7, 16, 17, 40], [0, 0, 0, 0, 0]),
    (dict(), [5, 33, 64], [11, 0, 70]),
    (dict(num_q_heads=2, num_kv_heads=2, page_size=32), [50, 3], [0, 100]),     # G = 1
    (dict(num_q_heads=8, num_kv_heads=1, head_dim=64), [20, 90], [3, 0]),        # G = 8
    (dict(kv_format="fp8", page_size=64, head_dim=32), [70, 5, 128], [0, 64, 60]),
])
def test_matches_torch_sdpa(kw, q_lens, prefix):
    p = synth.make_prefill_inputs(cfg(**kw), seed=2, q_lens=q_lens, prefix=prefix, poison=True)
    out, _ = prefill_attention(p)
    np.testing.assert_allclose(out, torch_reference(p), rtol=0, atol=1e-12)


def test_later_keys_never_matter():
    p = synth.make_prefill_inputs(cfg(), seed=3, q_lens=[60], prefix=[10])
    c = p.cache
    t = 25                                   # position 35: keys 36 .. 69 are in the future
    out1, lse1 = prefill_attention(p, rows={0: [t]})
    P = c.page_size
    for j in range(36, 70):
        phys = c.block_table[0, j // P]
        c.k_cache[phys, :, j % P] = synth.f32_to_bf16_bits(np.full(c.head_dim, 7.0, np.float32))
        c.v_cache[phys, :, j % P] = synth.f32_to_bf16_bits(np.full(c.head_dim, -3.0, np.float32))
    out2, lse2 = prefill_attention(p, rows={0: [t]})
    assert np.array_equal(out1[t], out2[t]) and np.array_equal(lse1[t], lse2[t])


def test_chunk_equals_the_tail_of_a_whole_prompt():
    """A 40-token chunk after a 90-token prefix gives the same rows as the last 40 rows
    of a 130-token prompt over the same cache."""
    chunk = synth.make_prefill_inputs(cfg(), seed=4, q_lens=[40], prefix=[90])
    whole = copy.deepcopy(chunk)
    rng = np.random.default_rng(5)
    head = synth.f32_to_bf16_bits(rng.standard_normal((90,) + chunk.q.shape[1:], dtype=np.float32))
    whole.q = np.concatenate([head, chunk.q])
    whole.q_lens = np.array([130], np.int32)
    whole.cu_q = np.array([0, 130], np.int32)
    o1, l1 = prefill_attention(chunk)
    o2, l2 = prefill_attention(whole, rows={0: range(90, 130)})
    np.testing.assert_allclose(o1, o2[90:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2[90:], rtol=0, atol=1e-13)
