"""Pins of the oracle's block-sparse decode (CPU only), against things other than
the sparse code path itself:
- an all-ones mask reproduces the dense oracle exactly;
- masking pages equals deleting them: the same request with the masked pages taken
  out of its block table (and its length shortened), evaluated by torch's float64
  scaled_dot_product_attention on a dense copy of the cache;
- the pages holding the step's query tokens are attended whatever their mask bit;
- closed form: with equal keys the output is the mean of V over the attended tokens.
"""

import copy

import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle_pins import small_cfg, torch_dense_reference


def sparse_cfgs():
    return [
        dict(batch=3, seq_lens=(40, 100, 161), page_size=16),
        dict(batch=2, seq_lens=(65, 200), q_len=4, page_size=16),              # draft rows
        dict(batch=2, seq_lens=(18, 49), q_len=4, page_size=16),               # draft spans 2 pages
        dict(batch=2, seq_lens=(130, 300), kv_format="fp8", page_size=64, q_len=2),
        dict(batch=2, seq_lens=(50, 97), num_q_heads=8, num_kv_heads=1, page_size=32),
    ]


@pytest.mark.parametrize("kw", sparse_cfgs())
def test_all_ones_mask_is_dense(kw):
    inp = synth.make_inputs(small_cfg(**kw), seed=4)
    ones = np.ones((inp.batch, inp.num_kv_heads, inp.block_table.shape[1]), np.uint8)
    o1, l1 = oracle.decode_attention(inp, block_mask=ones)
    o2, l2 = oracle.decode_attention(inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def removed_pages_input(inp, b, pages):
    """Request b's block table reduced to ``pages`` (in order) and its length
    shortened to the tokens they hold."""
    P = inp.page_size
    L = int(inp.seq_lens[b])
    sub = copy.deepcopy(inp)
    row = np.full(inp.block_table.shape[1], -1, np.int32)
    row[:len(pages)] = inp.block_table[b, pages]
    sub.block_table[b] = row
    sub.seq_lens[b] = sum(min(P, L - p * P) for p in pages)
    return sub


@pytest.mark.parametrize("kw", sparse_cfgs())
@pytest.mark.parametrize("keep", [0.0, 0.3, 0.7])
def test_masking_equals_deleting_pages(kw, keep):
    inp = synth.make_inputs(small_cfg(**kw), seed=5)
    mask = synth.make_block_mask(inp, keep, seed=6)
    out, lse = oracle.decode_attention(inp, block_mask=mask)
    G = inp.num_q_heads // inp.num_kv_heads
    att = synth.attended_pages(inp, mask)
    checked = 0
    for b in range(inp.batch):
        for g in range(inp.num_kv_heads):
            sub = removed_pages_input(inp, b, att[b][g])
            ref = torch_dense_reference(sub)                       # independent: torch SDPA
            sl = slice(g * G, (g + 1) * G)
            np.testing.assert_allclose(out[b, :, sl], ref[b, :, sl], rtol=0, atol=1e-12)
            checked += 1
    assert checked == inp.batch * inp.num_kv_heads


@pytest.mark.parametrize("kw", sparse_cfgs()[1:3])
def test_query_pages_are_always_attended(kw):
    inp = synth.make_inputs(small_cfg(**kw), seed=7)
    mask = synth.make_block_mask(inp, 0.5, seed=8)
    cleared, setp = mask.copy(), mask.copy()
    P, Tq = inp.page_size, inp.q_len
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        for p in range((L - Tq) // P, (L + P - 1) // P):
            cleared[b, :, p] = 0
            setp[b, :, p] = 1
    o1, l1 = oracle.decode_attention(inp, block_mask=cleared)
    o2, l2 = oracle.decode_attention(inp, block_mask=setp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_equal_keys_give_mean_of_attended_values():
    inp = synth.make_inputs(small_cfg(batch=2, seq_lens=(70, 150), q_len=2), seed=9)
    inp.k_cache[:] = inp.k_cache[0, 0, 0]                 # every key the same
    mask = synth.make_block_mask(inp, 0.4, seed=10)
    out, _ = oracle.decode_attention(inp, block_mask=mask)
    V = oracle.formats.bf16_bits_to_f64(inp.v_cache)
    P, G = inp.page_size, inp.num_q_heads // inp.num_kv_heads
    att = synth.attended_pages(inp, mask)
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        for g in range(inp.num_kv_heads):
            for t in range(inp.q_len):
                pos = L - inp.q_len + t
                rows = [V[inp.block_table[b, j // P], g, j % P] for j in range(pos + 1) if j // P in att[b][g]]
                np.testing.assert_allclose(out[b, t, g * G:(g + 1) * G], np.mean(rows, axis=0)[None].repeat(G, 0),
                                           rtol=0, atol=1e-12)
