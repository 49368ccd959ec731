"""The seeded generator: determinism, chunk-independence of draws, the recorded
length sums, poisoning, and the e4m3fn encoder's rounding (CPU only)."""

import numpy as np

import synth
from oracle.formats import E4M3FN_TABLE


def test_deterministic_and_recorded_sums():
    a = synth.make_inputs(synth.TINY, seed=0)
    b = synth.make_inputs(synth.TINY, seed=0)
    for x, y in ((a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.block_table, b.block_table)):
        assert np.array_equal(x, y)
    for name, total in (("mixed", 942439), ("fp8_spec", 291803)):
        sl = synth.draw_seq_lens(synth.ALL[name], np.random.default_rng(0))
        assert int(sl.sum()) == total


def test_chunked_draw_equals_single_draw(monkeypatch):
    import synth.gen as g
    cfg = dict(synth.TINY)
    monkeypatch.setattr(g, "_CHUNK_ELEMS", 1 << 30)
    one = synth.make_inputs(cfg, seed=9)
    monkeypatch.setattr(g, "_CHUNK_ELEMS", 3 * 16 * 64)
    many = synth.make_inputs(cfg, seed=9)
    assert np.array_equal(one.k_cache, many.k_cache) and np.array_equal(one.v_cache, many.v_cache)


def test_block_table_is_a_permutation():
    inp = synth.make_inputs(synth.TINY, seed=0, slack_pages=5)
    used = inp.block_table[inp.block_table >= 0]
    assert len(np.unique(used)) == len(used) == 29
    assert used.max() < inp.num_pages


def test_poison_touches_only_unused_elements():
    clean = synth.make_inputs(synth.TINY, seed=0, slack_pages=2)
    bad = synth.make_inputs(synth.TINY, seed=0, slack_pages=2, poison=True)
    diff = clean.k_cache != bad.k_cache
    assert diff.any()
    for b in range(clean.batch):
        L = int(clean.seq_lens[b])
        for j in range(L):
            phys = clean.block_table[b, j // 16]
            assert not diff[phys, :, j % 16].any()


def test_e4m3fn_encoder_is_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 100, rng.standard_normal(2000) * 0.01,
                        E4M3FN_TABLE[:126] , (E4M3FN_TABLE[:125] + E4M3FN_TABLE[1:126]) / 2, [500.0, -1e9, 0.0]])
    codes = synth.f32_to_e4m3fn(x)
    dec = E4M3FN_TABLE[codes]
    finite = E4M3FN_TABLE[np.isfinite(E4M3FN_TABLE)]
    for xi, di, ci in zip(x, dec, codes):
        xc = np.clip(xi, -448, 448)
        best = np.abs(finite - xc).min()
        assert abs(di - xc) == best
        if abs(abs(di - xc) - best) == 0 and np.sum(np.abs(finite - xc) == best) > 2:
            assert ci % 2 == 0


def test_algorithmic_bytes_of_mixed_workload():
    # K+V of every valid token + Q + out + block-table entries + seq_lens (see recipe)
    sl = synth.draw_seq_lens(synth.MIXED, np.random.default_rng(0)).astype(np.int64)
    pages = int(((sl + 15) // 16).sum())
    expect = int(sl.sum()) * 8 * 128 * 2 * 2 + 2 * 128 * 32 * 128 * 2 + 4 * pages + 4 * 128
    assert expect == 3862563668
