"""Pins of the fp64 oracle against things other than itself (CPU only).

- a library special case: torch's scaled_dot_product_attention in float64 on a
  dense copy of the cache built by an inverse page map, with torch's own bf16 and
  float8_e4m3fn decoders (GQA by repeat_interleave, an explicit causal mask);
- closed forms: one key gives v0; equal keys give the mean of V; a hand-worked
  three-key case;
- invariants: probabilities sum to 1, split + log-sum-exp merge equals the unsplit
  result, page-table permutation leaves the result unchanged, a draft row equals a
  one-token decode over the shorter prefix;
- the number-format tables against torch's conversions on every code.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.formats import E4M3FN_TABLE, bf16_bits_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(**kw):
    base = dict(name="t", batch=3, seq_lens=(5, 33, 70), q_len=1, num_q_heads=4,
                num_kv_heads=2, head_dim=16, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def torch_dense_reference(inp):
    """Independent reference: dense gather through the inverse page map, torch
    decoders, and torch SDPA in float64."""
    B, Tq, Hq, Hkv = inp.batch, inp.q_len, inp.num_q_heads, inp.num_kv_heads
    D, P = inp.head_dim, inp.page_size
    G = Hq // Hkv
    Lmax = int(inp.seq_lens.max())
    npg = (Lmax + P - 1) // P
    owner = {}
    for b in range(B):
        n = (int(inp.seq_lens[b]) + P - 1) // P
        for p in range(n):
            owner[int(inp.block_table[b, p])] = (b, p)

    def decode(cache, scales):
        if inp.kv_format == "bf16":
            t = torch.from_numpy(cache.view(np.int16).copy()).view(torch.bfloat16).double()
        else:
            t = torch.from_numpy(cache.copy()).view(torch.float8_e4m3fn).double()
            t = t * torch.from_numpy(scales.astype(np.float64))[:, :, None, None]
        return t

    kd = decode(inp.k_cache, inp.k_scale)
    vd = decode(inp.v_cache, inp.v_scale)
    K = torch.zeros(B, Hkv, npg * P, D, dtype=torch.float64)
    V = torch.zeros(B, Hkv, npg * P, D, dtype=torch.float64)
    for phys, (b, p) in owner.items():
        K[b, :, p * P:(p + 1) * P] = kd[phys]
        V[b, :, p * P:(p + 1) * P] = vd[phys]
    K = torch.nan_to_num(K[:, :, :Lmax])
    V = torch.nan_to_num(V[:, :, :Lmax])
    q = torch.from_numpy(inp.q.view(np.int16).copy()).view(torch.bfloat16).double()
    q = q.permute(0, 2, 1, 3)                                  # [B, Hq, Tq, D]
    Kr = K.repeat_interleave(G, dim=1)
    Vr = V.repeat_interleave(G, dim=1)
    j = torch.arange(Lmax)
    mask = torch.zeros(B, 1, Tq, Lmax, dtype=torch.bool)
    for b in range(B):
        L = int(inp.seq_lens[b])
        for t in range(Tq):
            mask[b, 0, t] = j <= L - Tq + t
    scale = float(np.float32(inp.scale))
    out = torch.nn.functional.scaled_dot_product_attention(q, Kr, Vr, attn_mask=mask, scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("kw", [
    dict(),
    dict(num_q_heads=2, num_kv_heads=2),                          # G = 1: plain MHA
    dict(q_len=4, seq_lens=(4, 17, 66)),                          # causal draft rows
    dict(kv_format="fp8", page_size=64, seq_lens=(64, 65, 130), q_len=2),
    dict(kv_format="fp8", page_size=16, seq_lens=(15, 17, 130), q_len=3),   # a scale per 16-token page
    dict(head_dim=64, page_size=32, num_q_heads=8, num_kv_heads=1),
])
def test_matches_torch_sdpa(kw):
    inp = synth.make_inputs(small_cfg(**kw), seed=3, poison=True, slack_pages=2)
    out, lse = oracle.decode_attention(inp)
    ref = torch_dense_reference(inp)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_large_magnitude_scores_match_sdpa():
    inp = synth.make_inputs(small_cfg(seq_lens=(40, 200, 9)), seed=5)
    q = bf16_bits_to_f64(inp.q) * 30.0
    inp.q = synth.f32_to_bf16_bits(q.astype(np.float32))
    out, _ = oracle.decode_attention(inp)
    np.testing.assert_allclose(out, torch_dense_reference(inp), rtol=0, atol=1e-11)


def test_single_key_gives_v0():
    inp = synth.make_inputs(small_cfg(seq_lens=(1, 1, 1)), seed=1)
    out, lse = oracle.decode_attention(inp)
    for b in range(3):
        phys = inp.block_table[b, 0]
        for h in range(4):
            v0 = bf16_bits_to_f64(inp.v_cache[phys, h // 2, 0])
            assert np.array_equal(out[b, 0, h], v0)


def test_equal_keys_give_mean_of_v():
    cfg = small_cfg(q_len=3, seq_lens=(3, 20, 47))
    inp = synth.make_inputs(cfg, seed=2)
    inp.k_cache[:] = inp.k_cache[0, 0, 0]          # every key identical
    out, _ = oracle.decode_attention(inp)
    for b in range(3):
        L = int(inp.seq_lens[b])
        for g in range(2):
            V = oracle.gather_kv(inp.v_cache, None, inp.block_table[b], L, g, 16, "bf16")
            for t in range(3):
                pos = L - 3 + t
                np.testing.assert_allclose(out[b, t, 2 * g:2 * g + 2], np.broadcast_to(V[:pos + 1].mean(0), (2, 16)),
                                           rtol=0, atol=1e-14)


def test_hand_worked_three_keys():
    """Golden case derived by hand (the pages print no numeric example)."""
    with open(os.path.join(GOLDEN, "three_keys.json")) as f:
        g = json.load(f)
    cfg = small_cfg(batch=1, seq_lens=(3,), num_q_heads=1, num_kv_heads=1, head_dim=2, page_size=16)
    inp = synth.make_inputs(cfg, seed=0)
    inp.q[:] = synth.f32_to_bf16_bits(np.array(g["q"], np.float32)).reshape(1, 1, 1, 2)
    inp.k_cache[:] = 0
    inp.v_cache[:] = 0
    phys = inp.block_table[0, 0]
    inp.k_cache[phys, 0, :3] = synth.f32_to_bf16_bits(np.array(g["k"], np.float32))
    inp.v_cache[phys, 0, :3] = synth.f32_to_bf16_bits(np.array(g["v"], np.float32))
    inp.scale = g["scale"]
    out, lse = oracle.decode_attention(inp)
    e = math.e
    expect = [(g["v"][0][d] + e * g["v"][1][d] + e * e * g["v"][2][d]) / (1 + e + e * e) for d in range(2)]
    np.testing.assert_allclose(out[0, 0, 0], expect, rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - math.log(1 + e + e * e)) < 1e-15


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(0)
    for L in (1, 7, 1000):
        K = rng.standard_normal((L, 32))
        p = oracle.attention.attention_probs(rng.standard_normal(32) * 5, K, 0.3)
        assert abs(p.sum() - 1.0) < 1e-12 and (p >= 0).all()


@pytest.mark.parametrize("q_len", [1, 4])
def test_split_then_merge_equals_unsplit(q_len):
    cfg = small_cfg(q_len=q_len, seq_lens=(9, 130, 301))
    inp = synth.make_inputs(cfg, seed=7)
    out, lse = oracle.decode_attention(inp)
    rng = np.random.default_rng(1)
    q = bf16_bits_to_f64(inp.q)
    for b in range(3):
        L = int(inp.seq_lens[b])
        for g in range(2):
            K = oracle.gather_kv(inp.k_cache, None, inp.block_table[b], L, g, 16, "bf16")
            V = oracle.gather_kv(inp.v_cache, None, inp.block_table[b], L, g, 16, "bf16")
            for t in range(q_len):
                pos = L - q_len + t
                for _ in range(3):
                    n_parts = rng.integers(1, 6)
                    lab = rng.integers(0, n_parts, pos + 1)
                    parts = [partial_for(q[b, t, 2 * g:2 * g + 2], K, V, inp.scale, np.nonzero(lab == i)[0])
                             for i in range(n_parts)]
                    o, l = oracle.lse_merge([p[0] for p in parts], [p[1] for p in parts])
                    np.testing.assert_allclose(o, out[b, t, 2 * g:2 * g + 2], rtol=0, atol=1e-12)
                    np.testing.assert_allclose(l, lse[b, t, 2 * g:2 * g + 2], rtol=0, atol=1e-12)


def partial_for(qrows, K, V, scale, idx):
    return oracle.partial_attention(qrows, K, V, float(np.float32(scale)), idx)


def test_merge_identities():
    rng = np.random.default_rng(2)
    o = rng.standard_normal((3, 5, 8))
    same = np.zeros((3, 5))
    m, l = oracle.lse_merge(o, same)
    np.testing.assert_allclose(m, o.mean(0), atol=1e-15)
    np.testing.assert_allclose(l, np.log(3.0), atol=1e-15)
    dom = np.array([[0.0] * 5, [80.0] * 5, [1.0] * 5])
    m, _ = oracle.lse_merge(o, dom)
    np.testing.assert_allclose(m, o[1], atol=1e-30)
    empty = np.full((2, 5), -np.inf)
    m, l = oracle.lse_merge(o[:2], empty)
    assert (m == 0).all() and np.isneginf(l).all()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_page_permutation_invariance(fmt):
    cfg = small_cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2, seq_lens=(70, 129, 3))
    inp = synth.make_inputs(cfg, seed=11, slack_pages=3)
    out, lse = oracle.decode_attention(inp)
    perm = np.random.default_rng(5).permutation(inp.num_pages)      # new position of page p
    inv = np.argsort(perm)
    inp.k_cache = inp.k_cache[inv]
    inp.v_cache = inp.v_cache[inv]
    if fmt == "fp8":
        inp.k_scale = inp.k_scale[inv]
        inp.v_scale = inp.v_scale[inv]
    bt = inp.block_table.copy()
    inp.block_table = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    out2, lse2 = oracle.decode_attention(inp)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_draft_row_equals_shorter_single_token_decode():
    cfg = small_cfg(q_len=4, seq_lens=(4, 17, 50))
    inp = synth.make_inputs(cfg, seed=4)
    out, lse = oracle.decode_attention(inp)
    for t in range(4):
        one = synth.make_inputs(small_cfg(q_len=1, seq_lens=(4, 17, 50)), seed=4)
        one.k_cache, one.v_cache, one.block_table = inp.k_cache, inp.v_cache, inp.block_table
        one.q = inp.q[:, t:t + 1].copy()
        one.seq_lens = (inp.seq_lens - 4 + t + 1).astype(np.int32)
        o1, l1 = oracle.decode_attention(one)
        assert np.array_equal(o1[:, 0], out[:, t]) and np.array_equal(l1[:, 0], lse[:, t])


def test_e4m3fn_table_matches_torch():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(E4M3FN_TABLE))
    assert np.array_equal(ref[~nan], E4M3FN_TABLE[~nan])
    assert nan.sum() == 2 and E4M3FN_TABLE[0x7E] == 448.0


def test_bf16_decoder_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and np.array_equal(ref[~nan], got[~nan])
