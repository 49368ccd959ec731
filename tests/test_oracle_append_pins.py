"""Pins of the fused KV-append oracle (CPU only), against things other than itself:
- the e4m3fn encoder against torch's float8_e4m3fn conversion on in-range values
  (random values, every grid midpoint, subnormals), every code round-tripping, and
  hand-worked saturation and sign cases;
- the bf16 rounding against torch's float32 -> bfloat16 conversion;
- the rotation: closed forms (identity, quarter turn), norm preservation, and a float64
  complex rotation within float32 rounding;
- the append: bf16 rows copied bit for bit to the right pages and offsets, nothing else
  touched; a fresh fp8 page written whole equals the generator's independent tile
  quantisation; the keep-scale and re-encode branches by hand-checkable properties.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import append as A
from oracle.formats import E4M3FN_TABLE, bf16_bits_to_f64


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_round_trips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = E4M3FN_TABLE[codes].astype(np.float32)
    got = A.encode_e4m3fn(vals)
    # -0.0 (0x80) decodes to -0.0 and must come back as 0x80; every other code likewise
    assert np.array_equal(got, codes)


def test_encoder_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-448, 448, 100000).astype(np.float32),
        (rng.standard_normal(100000) * 2.0 ** -8).astype(np.float32),      # subnormal range
    ])
    grid = E4M3FN_TABLE[:0x7F]
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)                 # exact in float32
    x = np.concatenate([x, mids, -mids, grid.astype(np.float32)])
    x = x[np.abs(x) <= 448]
    got = A.encode_e4m3fn(x)
    want = torch_e4m3(x)
    zero = (want & 0x7F) == 0              # torch may drop the sign of a value rounding to 0
    assert np.array_equal(got[~zero], want[~zero])
    assert np.array_equal(got[zero] & 0x7F, want[zero] & 0x7F)


def test_encoder_saturates_and_keeps_sign():
    x = np.array([448, 449, 463.9, 464, 500, 1e30, np.inf, -448, -1000, -np.inf,
                  -0.0, -1e-9, 1e-9, 2.0 ** -10, 2.0 ** -10 * 3], np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE,
            0x80, 0x80, 0x00, 0x00, 0x02]   # 2^-10 ties to 0 (even); 3 * 2^-10 ties to 2 * 2^-9
    assert A.encode_e4m3fn(x).tolist() == want


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300000) * 10.0 ** rng.uniform(-5, 5, 300000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(A.f32_to_bf16_bits_rne(x), want)


def test_rotation_closed_forms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    one, zero = np.ones((5, 32), np.float32), np.zeros((5, 32), np.float32)
    assert np.array_equal(A.rope_half(x, one, zero), x)
    quarter = A.rope_half(x, zero, one)
    assert np.array_equal(quarter[:, :32], -x[:, 32:]) and np.array_equal(quarter[:, 32:], x[:, :32])


def test_rotation_matches_complex_multiplication():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((100, 128)).astype(np.float32)
    ang = rng.uniform(-100, 100, (100, 64))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    got = A.rope_half(x, c, s).astype(np.float64)
    z = (x[:, :64].astype(np.float64) + 1j * x[:, 64:]) * (c.astype(np.float64) + 1j * s)
    ref = np.concatenate([z.real, z.imag], axis=1)
    # each output is two float32 products and one float32 sum: within 3 ulp of the terms
    bound = 3 * 2.0 ** -24 * (np.abs(x[:, :64]) + np.abs(x[:, 64:])).repeat(2, axis=0).reshape(100, 128)
    assert (np.abs(got - ref) <= bound + 1e-30).all()
    n_in = np.hypot(x[:, :64], x[:, 64:])
    n_out = np.hypot(got[:, :64], got[:, 64:])
    np.testing.assert_allclose(n_out, n_in * np.hypot(c, s), rtol=1e-6)


def small_inputs(fmt, q_len=2, P=16, seed=4, lens=(5, 16, 17, 40)):
    c = dict(name="a", batch=len(lens), seq_lens=lens, q_len=q_len, num_q_heads=4, num_kv_heads=2,
             head_dim=64, page_size=P, kv_format=fmt)
    return synth.make_inputs(c, seed=seed, slack_pages=2)


def new_rows(inp, seed=5, scale=1.0):
    rng = np.random.default_rng(seed)
    shape = (inp.batch, inp.q_len, inp.num_kv_heads, inp.head_dim)
    k = synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    v = synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))
    return k, v


def test_bf16_append_copies_rows_and_touches_nothing_else():
    inp = small_inputs("bf16", q_len=3)
    k_new, v_new = new_rows(inp)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    A.kv_append(kc, vc, None, None, inp.block_table, inp.seq_lens, k_new, v_new)
    ek, ev = inp.k_cache.copy(), inp.v_cache.copy()
    P = inp.page_size
    for b in range(inp.batch):
        L = int(inp.seq_lens[b])
        for t in range(inp.q_len):
            pos = L - inp.q_len + t
            ek[inp.block_table[b, pos // P], :, pos % P] = k_new[b, t]
            ev[inp.block_table[b, pos // P], :, pos % P] = v_new[b, t]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_fresh_fp8_page_written_whole_equals_tile_quantisation():
    """64 new tokens filling a fresh page at once: the generator's independent encoder
    (frexp-based) with its own amax / 448 scale gives the same values."""
    inp = small_inputs("fp8", q_len=1, P=64, lens=(64, 128))
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 64, 2, 64)).astype(np.float32)
    kb = synth.f32_to_bf16_bits(x)
    xf = bf16_bits_to_f64(kb).astype(np.float32)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    ks, vs = inp.k_scale.copy(), inp.v_scale.copy()
    A.kv_append(kc, vc, ks, vs, inp.block_table, inp.seq_lens, kb, kb, kv_format="fp8")
    for b in range(2):
        phys = inp.block_table[b, (int(inp.seq_lens[b]) - 1) // 64]
        for g in range(2):
            rows = xf[b, :, g]
            s = np.float32(np.abs(rows).max() / np.float32(448))
            assert ks[phys, g] == s and vs[phys, g] == s
            want = E4M3FN_TABLE[synth.f32_to_e4m3fn(rows / s)]
            assert np.array_equal(E4M3FN_TABLE[kc[phys, g]], want)


def test_fp8_small_values_keep_the_scale_and_old_codes():
    inp = small_inputs("fp8", q_len=2, P=64, lens=(30, 100))
    k_new, v_new = new_rows(inp, scale=0.01)          # far inside every page's range
    kc, ks = inp.k_cache.copy(), inp.k_scale.copy()
    A.kv_append(kc, inp.v_cache.copy(), ks, inp.v_scale.copy(), inp.block_table, inp.seq_lens,
                k_new, v_new, kv_format="fp8")
    assert np.array_equal(ks, inp.k_scale)
    for b in range(2):
        L = int(inp.seq_lens[b])
        phys = inp.block_table[b, (L - 2) // 64]
        o = (L - 2) % 64
        assert np.array_equal(kc[phys, :, :o], inp.k_cache[phys, :, :o])


def test_fp8_large_values_raise_the_scale_and_reencode():
    inp = small_inputs("fp8", q_len=1, P=64, lens=(30, 100))
    k_new, v_new = new_rows(inp, scale=1e4)           # beyond every page's range
    kc, ks = inp.k_cache.copy(), inp.k_scale.copy()
    A.kv_append(kc, inp.v_cache.copy(), ks, inp.v_scale.copy(), inp.block_table, inp.seq_lens,
                k_new, v_new, kv_format="fp8")
    for b in range(2):
        L = int(inp.seq_lens[b])
        phys = inp.block_table[b, (L - 1) // 64]
        o = (L - 1) % 64
        for g in range(2):
            s_old, s_new = inp.k_scale[phys, g], ks[phys, g]
            new_amax = np.abs(bf16_bits_to_f64(k_new[b, 0, g])).max()
            assert s_new == np.float32(np.float32(new_amax) / np.float32(448)) and s_new > s_old
            old = E4M3FN_TABLE[inp.k_cache[phys, g, :o]] * np.float64(s_old)
            new = E4M3FN_TABLE[kc[phys, g, :o]] * np.float64(s_new)
            # re-encoding moves an old value by at most half a step of the new grid
            # (steps are 2^-9 * s_new below 2^-6 * s_new, else 1/16 of the value)
            step = np.maximum(np.abs(old) / 8, 2.0 ** -9 * s_new)
            assert (np.abs(new - old) <= step / 2 + 1e-12).all()
