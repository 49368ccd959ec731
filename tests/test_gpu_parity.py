"""GPU parity of the HIP decode path against the fp64 oracle (needs an MI355X).

Tolerances (the contract): max |gpu - oracle| <= 1e-2 on the bf16 output for BF16 KV
and <= 3e-2 for FP8 KV, against the oracle on the same stored inputs. One exception
is forced by the output format: a bf16 value of magnitude >= 4 has a spacing of
2^-5, so rounding alone can move it 1.6e-2; there the bound is 0.6 bf16 ulp of the
reference instead (elementwise tolerance max(tol, 0.6 * ulp_bf16(ref))).

Tighter diagnostics are asserted too, because an absolute 1e-2 is loose at long L
(outputs shrink like 1/sqrt(L)): relative L2 error <= 1e-2 and |lse - lse_ref| <= 1e-3.
The arithmetic behind them: bf16 weights (relative 2^-9 each, averaging out), fp32
accumulation, one bf16 rounding of the output (2^-9 relative).
"""

import numpy as np
import pytest

import oracle
import synth
from oracle.formats import E4M3FN_TABLE, bf16_bits_to_f64
from tests.gpu_util import (device_inputs, log, make_runner, max_abs, pages_past_two_gib, rel_l2,
                            run_decode)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp8": 3e-2}
REL_TOL = 1e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def cfg(**kw):
    base = dict(name="case", batch=0, seq_lens=(1,), q_len=1, num_q_heads=8, num_kv_heads=2,
                head_dim=128, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    _, e = np.frexp(np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


def excess(out, ref, tol):
    """Largest amount by which |out - ref| exceeds the elementwise tolerance."""
    err = np.abs(np.asarray(out, np.float64) - ref)
    return float(np.max(err - np.maximum(tol, 0.6 * bf16_ulp(ref)), initial=-np.inf))


def ulp_branch(out, ref, tol):
    """Elements whose bound is the 0.6-ulp one (it exceeds the flat tolerance) and
    the largest error among them, as (count, max_abs)."""
    ref = np.asarray(ref, np.float64)
    sel = 0.6 * bf16_ulp(ref) > tol
    if not sel.any():
        return 0, 0.0
    return int(sel.sum()), float(np.max(np.abs(np.asarray(out, np.float64)[sel] - ref[sel])))


def check(inp, out, lse, pairs=None, tag="", block_mask=None):
    ref_out, ref_lse = oracle.decode_attention(inp, pairs=pairs, block_mask=block_mask)
    if pairs is not None:
        sel = np.zeros(ref_lse.shape, dtype=bool)
        G = inp.num_q_heads // inp.num_kv_heads
        for b, g in pairs:
            sel[b, :, g * G:(g + 1) * G] = True
        out, ref_out = out[sel], ref_out[sel]
        lse, ref_lse = lse[sel], ref_lse[sel]
    assert np.isfinite(out).all() and np.isfinite(lse).all(), tag
    tol = TOL[inp.kv_format]
    ea, er, el = max_abs(out, ref_out), rel_l2(out, ref_out), max_abs(lse, ref_lse)
    nu, eu = ulp_branch(out, ref_out, tol)
    log("  %s: %d outputs, max_abs %.3e rel_l2 %.3e lse %.3e; ulp branch %d outputs, max_abs %.3e"
        % (tag, np.size(out), ea, er, el, nu, eu))
    assert excess(out, ref_out, tol) <= 0, tag
    assert er <= REL_TOL, tag
    assert el <= LSE_TOL, tag


SMALL = [
    dict(id="tiny_auto", c=synth.TINY, T=0, W=0),
    dict(id="tiny_T16_W1", c=synth.TINY, T=16, W=1),
    dict(id="tiny_T64_W3", c=synth.TINY, T=64, W=3),
    dict(id="g4_d128_p16", c=cfg(), sl=[1, 15, 16, 17, 33, 100, 257, 700], T=64, W=7),
    dict(id="g4_d128_p16_T48", c=cfg(), sl=[31, 32, 47, 48, 49, 95, 96, 97], T=48, W=3),
    dict(id="g8_d128_p64", c=cfg(num_q_heads=16, page_size=64), sl=[63, 64, 65, 500, 1000], T=128, W=5),
    dict(id="g1_d64_p32", c=cfg(num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=32),
         sl=[3, 90, 333], T=32, W=2),
    dict(id="g16_d128", c=cfg(num_q_heads=16, num_kv_heads=1), sl=[40, 300, 2049], T=256, W=3),
    dict(id="spec4_g4", c=cfg(q_len=4), sl=[4, 5, 6, 7, 33, 34, 35, 129], T=32, W=4),
    dict(id="spec2_g8_d64", c=cfg(q_len=2, num_q_heads=16, head_dim=64), sl=[2, 17, 48, 49], T=16, W=3),
    dict(id="spec3_g4_auto", c=cfg(q_len=3), sl=[3, 300, 1000, 4097], T=0, W=11),
    dict(id="fp8_spec4", c=cfg(kv_format="fp8", page_size=64, q_len=4),
         sl=[4, 64, 65, 66, 67, 200, 513], T=64, W=5),
    dict(id="fp8_d64", c=cfg(kv_format="fp8", page_size=64, num_q_heads=4, num_kv_heads=1, head_dim=64),
         sl=[1, 100, 1000], T=128, W=2),
    dict(id="fp8_auto_g8", c=cfg(kv_format="fp8", page_size=64, num_q_heads=16, q_len=2),
         sl=[2, 777, 3000, 64 * 65 + 1], T=0, W=9),
    dict(id="g4_d128_p48", c=cfg(page_size=48), sl=[1, 47, 48, 49, 95, 200, 1000], T=96, W=5),
    dict(id="spec2_g8_d64_p48_auto", c=cfg(page_size=48, num_q_heads=16, head_dim=64, q_len=2),
         sl=[2, 48, 97, 2000, 4801], T=0, W=9),
    dict(id="fp8_d64_spec4_g4", c=cfg(kv_format="fp8", page_size=64, head_dim=64, q_len=4),
         sl=[4, 5, 63, 64, 65, 67, 130, 1000, 4097], T=128, W=6),
    # More than 16 rows per kv head (two or four MFMA column blocks):
    dict(id="g8_spec3_m24", c=cfg(num_q_heads=16, q_len=3), sl=[3, 4, 17, 33, 100, 1000], T=64, W=5),
    dict(id="g8_spec4_m32", c=cfg(num_q_heads=16, q_len=4), sl=[4, 5, 6, 7, 64, 65, 300, 2049], T=0, W=7),
    dict(id="g5_spec4_m20_p48", c=cfg(num_q_heads=10, page_size=48, q_len=4), sl=[4, 47, 48, 49, 500],
         T=96, W=3),
    dict(id="g16_spec4_m64", c=cfg(num_q_heads=32, q_len=4), sl=[4, 5, 6, 7, 35, 129, 777, 3000], T=64, W=6),
    dict(id="g12_spec3_m36_d64", c=cfg(num_q_heads=24, head_dim=64, q_len=3), sl=[3, 16, 31, 250, 1500],
         T=0, W=5),
    dict(id="g16_spec3_m48_p32", c=cfg(num_q_heads=32, page_size=32, q_len=3), sl=[3, 32, 33, 97, 2000],
         T=128, W=4),
    dict(id="g64_m64", c=cfg(num_q_heads=64, num_kv_heads=1), sl=[1, 2, 100, 5000], T=256, W=9),
    dict(id="g32_spec2_m64_d64_p64", c=cfg(num_q_heads=64, num_kv_heads=2, head_dim=64, page_size=64, q_len=2),
         sl=[2, 64, 65, 1234], T=0, W=4),
    dict(id="fp8_g8_spec4_m32", c=cfg(kv_format="fp8", page_size=64, num_q_heads=16, q_len=4),
         sl=[4, 64, 65, 66, 67, 200, 2049], T=64, W=5),
    dict(id="fp8_g16_spec4_m64", c=cfg(kv_format="fp8", page_size=64, num_q_heads=32, q_len=4),
         sl=[4, 5, 64, 67, 129, 1000, 4097], T=0, W=6),
    dict(id="fp8_g16_spec3_m48_d64", c=cfg(kv_format="fp8", page_size=64, head_dim=64, num_q_heads=32, q_len=3),
         sl=[3, 66, 700, 3001], T=128, W=3),
    dict(id="fp8_g12_spec2_m24", c=cfg(kv_format="fp8", page_size=64, num_q_heads=24, q_len=2),
         sl=[2, 63, 64, 65, 1500], T=0, W=4),
    # FP8 with pages shorter than 64 tokens (one scale per page; a 32-token chunk
    # spans two 16-token pages) and pages not aligned to chunks (48):
    dict(id="fp8_p16_spec4", c=cfg(kv_format="fp8", page_size=16, q_len=4),
         sl=[4, 15, 16, 17, 33, 100, 257, 1000], T=64, W=7),
    dict(id="fp8_p32_g8_spec2", c=cfg(kv_format="fp8", page_size=32, num_q_heads=16, q_len=2),
         sl=[2, 31, 32, 33, 500, 2049], T=0, W=5),
    dict(id="fp8_p48_d64", c=cfg(kv_format="fp8", page_size=48, head_dim=64),
         sl=[1, 47, 48, 49, 95, 97, 700], T=192, W=3),
    dict(id="fp8_p16_g16_spec4_m64", c=cfg(kv_format="fp8", page_size=16, num_q_heads=32, q_len=4),
         sl=[4, 17, 64, 129, 1500], T=128, W=4),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["id"] for c in SMALL])
def test_small_cases_match_oracle(case):
    c = dict(case["c"])
    inp = synth.make_inputs(c, seed=17, poison=True, slack_pages=3, seq_lens=case.get("sl"))
    log("case %s B=%d Tq=%d G=%d D=%d P=%d %s T=%d W=%d" % (
        case["id"], inp.batch, inp.q_len, inp.num_q_heads // inp.num_kv_heads, inp.head_dim,
        inp.page_size, inp.kv_format, case["T"], case["W"]))
    out, lse, _ = run_decode(inp, case["T"], case["W"])
    check(inp, out, lse, tag=case["id"])


def random_case(seed):
    """A small random decode batch from ``default_rng(seed)``: head group and draft
    tokens (up to 64 rows per kv head), kv heads, head dim, page size, format, lengths,
    a fixed tile (a multiple of the format's quantum) or the automatic one, workers."""
    rng = np.random.default_rng(2000 + seed)
    Tq = int(rng.integers(1, 5))
    G = int(rng.choice([g for g in (1, 2, 3, 4, 5, 8, 12, 16, 32, 64) if g * Tq <= 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([16, 32, 48, 64]))
    fmt = str(rng.choice(["bf16", "fp8"]))
    c = cfg(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=int(rng.choice([64, 128])),
            page_size=P, kv_format=fmt, q_len=Tq)
    B = int(rng.integers(1, 9))
    sl = [int(x) for x in rng.integers(Tq, 3000, B)]
    quantum = P if fmt == "bf16" else P * 64 // int(np.gcd(P, 64))
    T = 0 if rng.random() < 0.3 else quantum * int(rng.integers(1, 9))
    W = int(rng.integers(1, 13))
    return c, sl, T, W


@pytest.mark.parametrize("seed", range(16))
def test_random_small_shapes_match_oracle(seed):
    c, sl, T, W = random_case(seed)
    inp = synth.make_inputs(c, seed=40 + seed, poison=True, slack_pages=2, seq_lens=sl)
    tag = "random %d: B=%d Tq=%d G=%d Hkv=%d D=%d P=%d %s T=%d W=%d" % (
        seed, inp.batch, inp.q_len, inp.num_q_heads // inp.num_kv_heads, inp.num_kv_heads,
        inp.head_dim, inp.page_size, inp.kv_format, T, W)
    log(tag)
    out, lse, _ = run_decode(inp, T, W)
    check(inp, out, lse, tag=tag)


@pytest.mark.parametrize("name", ["llama8b", "mixed", "long", "fp8_spec"])
def test_full_size_workloads(name):
    """The full workloads in the launch configuration the bench times (automatic tile
    size, default worker count); every (request, kv head) group against the oracle."""
    import torch
    log("full-size %s: generating inputs" % name)
    inp = synth.make_inputs(synth.ALL[name], seed=0)
    log("full-size %s: running" % name)
    out, lse, _ = run_decode(inp)
    log("full-size %s: oracle over all %d groups" % (name, inp.batch * inp.num_kv_heads))
    check(inp, out, lse, tag=name)
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,q_len,heads", [("long", 4, (64, 8)), ("fp8_spec", 4, (64, 4))])
def test_full_size_wide_groups(name, q_len, heads):
    """A workload's shape with more than 16 rows per kv head: the long workload's
    64 q / 8 kv heads with four draft tokens (32 rows), and the fp8 workload with 64 q /
    4 kv heads (64 rows) at 8 requests; default launch, every group against the oracle."""
    import torch
    c = dict(synth.ALL[name], q_len=q_len, num_q_heads=heads[0], num_kv_heads=heads[1])
    if name == "fp8_spec":
        c["batch"] = 8
    log("full-size wide %s: generating inputs" % name)
    inp = synth.make_inputs(c, seed=0)
    out, lse, _ = run_decode(inp)
    check(inp, out, lse, tag="%s Tq=%d %dq/%dkv" % ((name, q_len) + heads))
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("keys", [2, 3, 4])
@pytest.mark.parametrize("G", [1, 16, 64])
def test_few_key_rows_worst_rounding(keys, G):
    """Rows that see 2-4 keys with the inputs a float32 model of the kernel's rounding
    finds worst for bf16 weights (tests/decode_rounding.py): 64 requests of L = keys,
    q = e_0 in every query head, key j = a_j e_0, every head dim of value j = v_j.
    Without the low part of P these rows exceed the 1e-2 contract in the model; the
    kernel must meet it (G = 1, 16 take one MFMA column block, 64 four)."""
    from tests.decode_rounding import search_rows
    r = search_rows(float(1.0 / np.sqrt(128.0)), keys=keys, samples=300_000, seed=keys)
    n = len(r["a"])
    inp = synth.make_inputs(cfg(num_q_heads=G, num_kv_heads=1), seed=3, seq_lens=[keys] * n)
    inp.q[:] = 0
    inp.q[:, :, :, 0] = synth.f32_to_bf16_bits(np.float32(1.0))
    for i in range(n):
        page = inp.block_table[i, 0]
        inp.k_cache[page, 0, :keys, :] = 0
        inp.k_cache[page, 0, :keys, 0] = synth.f32_to_bf16_bits(r["a"][i].astype(np.float32))
        inp.v_cache[page, 0, :keys, :] = synth.f32_to_bf16_bits(r["v"][i].astype(np.float32))[:, None]
    log("few-key rows: %d keys, G=%d; model without the low part: worst error %.3e" % (
        keys, G, r["err_plain"].max()))
    out, lse, _ = run_decode(inp)
    assert (out == out[:, :, :1, :1]).all()     # every head and dim of a request agrees
    check(inp, out, lse, tag="few keys %d G %d" % (keys, G))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_million_token_request(fmt):
    """One request of 1 000 003 tokens beside a short one (two draft tokens each): tile
    indices up to 1M / T, host and device plans; every row is checked against the
    oracle."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = cfg(name="long1m", q_len=2, num_q_heads=4, num_kv_heads=1, kv_format=fmt,
            page_size=64 if fmt == "fp8" else 16)
    inp = synth.make_inputs(c, seed=41, seq_lens=[1_000_003, 17])
    log("million-token request %s: %d pages" % (fmt, inp.k_cache.shape[0]))
    dev = device_inputs(inp)
    out, lse, bits = run_decode(inp, dev=dev)
    check(inp, out, lse, tag="1M %s host plan" % fmt)
    r = pkv.PagedDecode(num_q_heads=4, num_kv_heads=1, head_dim=128, page_size=inp.page_size,
                        kv_format=fmt, q_len=2, device_plan=True)
    out_d, lse_d, bits_d = run_decode(inp, dev=dev, runner=r)
    assert r.plan_info()["status"] == 0
    assert np.array_equal(bits, bits_d) and np.array_equal(lse, lse_d)
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_pages_past_two_gib(fmt):
    """The same pages moved to physical indices whose byte offsets lie past 2^31 in a
    ~2.2 GB cache tensor (the rest of it NaN, never read): bit-identical to the compact
    cache."""
    import torch
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2)
    inp = synth.make_inputs(c, seed=43, seq_lens=[2, 300, 1000, 5000])
    dev = device_inputs(inp)
    _, lse_a, bits_a = run_decode(inp, dev=dev)
    moved, base, nbytes = pages_past_two_gib(inp, dev)
    log("pages past 2 GiB (%s): %.2f GB per cache tensor, first used page %d" % (fmt, nbytes / 1e9, base))
    _, lse_b, bits_b = run_decode(inp, dev=moved)
    assert np.array_equal(bits_a, bits_b) and np.array_equal(lse_a, lse_b)
    del moved, dev
    torch.cuda.empty_cache()


def medium_inputs(fmt="bf16", seed=5, **kw):
    c = cfg(num_q_heads=32, num_kv_heads=8, kv_format=fmt, page_size=64 if fmt == "fp8" else 16, **kw)
    sl = [1, 64, 300, 1023, 2500, 4096]
    return synth.make_inputs(c, seed=seed, slack_pages=5, seq_lens=[max(x, c["q_len"]) for x in sl])


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_bitwise_repeatable(fmt):
    inp = medium_inputs(fmt)
    dev = device_inputs(inp)
    _, l1, b1 = run_decode(inp, dev=dev)
    _, l2, b2 = run_decode(inp, dev=dev)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_page_permutation_is_bitwise_invariant(fmt):
    inp = medium_inputs(fmt, q_len=2)
    _, l1, b1 = run_decode(inp)
    perm = np.random.default_rng(3).permutation(inp.num_pages)
    inv = np.argsort(perm)
    inp.k_cache, inp.v_cache = inp.k_cache[inv], inp.v_cache[inv]
    if fmt == "fp8":
        inp.k_scale, inp.v_scale = inp.k_scale[inv], inp.v_scale[inv]
    bt = inp.block_table
    inp.block_table = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    _, l2, b2 = run_decode(inp)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_nan_poison_is_never_read(fmt):
    clean = medium_inputs(fmt, q_len=3)
    dirty = medium_inputs(fmt, q_len=3)
    synth.apply_poison(dirty)
    _, l1, b1 = run_decode(clean)
    _, l2, b2 = run_decode(dirty)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


def test_v_all_ones_gives_exactly_one():
    inp = medium_inputs("bf16")
    inp.v_cache[:] = 0x3F80
    out, _, _ = run_decode(inp, tile_tokens=256, num_workers=7)
    assert (out == 1.0).all()


def test_single_key_gives_v0_bit_exact():
    inp = synth.make_inputs(cfg(), seed=2, seq_lens=[1] * 9)
    _, _, bits = run_decode(inp)
    G = inp.num_q_heads // inp.num_kv_heads
    for b in range(inp.batch):
        for h in range(inp.num_q_heads):
            assert np.array_equal(bits[b, 0, h], inp.v_cache[inp.block_table[b, 0], h // G, 0])


@pytest.mark.parametrize("q_len", [1, 4])
def test_equal_keys_give_mean_of_v(q_len):
    inp = medium_inputs("bf16", q_len=q_len)
    inp.k_cache[:] = inp.k_cache[0, 0, 0]
    out, lse, _ = run_decode(inp, tile_tokens=128, num_workers=5)
    check(inp, out, lse, tag="equal keys")


def test_large_magnitude_scores():
    inp = medium_inputs("bf16", q_len=2)
    inp.q = synth.f32_to_bf16_bits((bf16_bits_to_f64(inp.q) * 30.0).astype(np.float32))
    out, lse, _ = run_decode(inp)
    ref_out, ref_lse = oracle.decode_attention(inp)
    assert np.isfinite(out).all()
    assert excess(out, ref_out, TOL["bf16"]) <= 0
    assert max_abs(lse, ref_lse) <= 30 * LSE_TOL     # lse scales with the scores


def test_draft_rows_match_single_token_decodes():
    sl = [4, 17, 33, 34, 35, 36, 100]
    inp = synth.make_inputs(cfg(q_len=4), seed=8, seq_lens=sl)
    out4, _, _ = run_decode(inp, tile_tokens=16, num_workers=3)
    for t in range(4):
        one = synth.make_inputs(cfg(q_len=1), seed=8, seq_lens=sl)
        one.k_cache, one.v_cache, one.block_table = inp.k_cache, inp.v_cache, inp.block_table
        one.q = inp.q[:, t:t + 1].copy()
        one.seq_lens = (inp.seq_lens - 4 + t + 1).astype(np.int32)
        out1, _, _ = run_decode(one, tile_tokens=16, num_workers=3)
        assert excess(out4[:, t], out1[:, 0].astype(np.float64), TOL["bf16"]) <= 0


def test_fp8_codes_decode_exactly():
    """Every finite e4m3fn code read through the kernel's V path with one key and
    scale 1 comes back as its exact value (decoded in bf16)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    inp = synth.make_inputs(cfg(kv_format="fp8", page_size=64, num_q_heads=1, num_kv_heads=1),
                            seed=1, seq_lens=[1, 1])
    inp.v_scale[:] = 1.0
    flat = np.zeros(256, dtype=np.uint8)
    flat[:len(codes)] = codes
    for b in range(2):
        inp.v_cache[inp.block_table[b, 0], 0, 0, :] = flat[128 * b:128 * (b + 1)]
    out, _, _ = run_decode(inp)
    got = out[:, 0, 0, :].reshape(-1)[:len(codes)]
    assert np.array_equal(got, E4M3FN_TABLE[codes])


@pytest.mark.parametrize("T,W", [(16, 1), (48, 13), (256, 512), (1024, 64), (4096, 2)])
def test_tile_and_worker_sweep(T, W):
    inp = medium_inputs("bf16", q_len=2)
    out, lse, _ = run_decode(inp, tile_tokens=T, num_workers=W)
    check(inp, out, lse, tag="T=%d W=%d" % (T, W))


def test_combine_alone_matches_lse_merge():
    import torch
    import paged_kv_gqa_amd as pkv
    rng = np.random.default_rng(4)
    B, Tq, Hq, Hkv, D = 3, 2, 8, 2, 128
    G, M = Hq // Hkv, (Hq // Hkv) * Tq
    nb = np.array([1, 4, 9], dtype=np.int32)
    rtb = np.concatenate([[0], np.cumsum(nb)]).astype(np.int32)
    NP = int(Hkv * rtb[-1])
    o = rng.standard_normal((NP, M, D)).astype(np.float32)
    lse = (rng.standard_normal((NP, M)) * 3).astype(np.float32)
    lse[5, 2] = -np.inf
    nbytes = pkv.pkv_workspace_bytes(NP, M, D)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    obytes = NP * M * D * 4
    ws[:obytes].copy_(torch.from_numpy(o.view(np.uint8).reshape(-1)))
    off = (obytes + 255) // 256 * 256
    ws[off:off + NP * M * 4].copy_(torch.from_numpy(lse.view(np.uint8).reshape(-1)))
    out = torch.empty((B, Tq, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse_out = torch.empty((B, Tq, Hq), dtype=torch.float32, device="cuda")
    pkv.pkv_combine(workspace=ws, workspace_bytes=nbytes, num_partials=NP,
                    req_tile_base=torch.from_numpy(rtb).cuda(), batch=B, q_len=Tq, num_q_heads=Hq,
                    num_kv_heads=Hkv, head_dim=D, out=out, lse_out=lse_out)
    torch.cuda.synchronize()
    got, got_lse = out.float().cpu().numpy(), lse_out.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            for h in range(Hq):
                g, r = h // G, t * G + h % G
                slots = Hkv * rtb[b] + g * nb[b] + np.arange(nb[b])
                ref, ref_l = oracle.lse_merge(o[slots, r], lse[slots, r])
                assert np.all(np.abs(got[b, t, h] - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
                assert abs(got_lse[b, t, h] - ref_l) <= 1e-5 * max(1.0, abs(ref_l))


@pytest.mark.parametrize("fmt,T", [("bf16", 4096), ("bf16", 256), ("fp8", 8192), ("fp8", 128)])
def test_single_tile_rows_written_by_decode_equal_the_combine(fmt, T):
    """With out / lse_out in the decode arguments, requests cut into one tile get their
    final rows from decode_partial itself: bit for bit what the combine writes from the
    same partials; rows of longer requests are left alone (sentinel kept)."""
    import torch
    import paged_kv_gqa_amd as pkv
    from tests.test_zz_no_alloc import step_args
    inp = medium_inputs(fmt, q_len=2)
    dev = device_inputs(inp)
    kw, _plan = step_args(inp, dev, T=T)
    M = (inp.num_q_heads // inp.num_kv_heads) * inp.q_len
    nbytes = pkv.pkv_workspace_bytes(max(kw["num_partials"], 1), M, inp.head_dim)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    shape = (inp.batch, inp.q_len, inp.num_q_heads)
    out_d = torch.full(shape + (inp.head_dim,), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_d = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
    pkv.pkv_decode_partial(workspace=ws, workspace_bytes=nbytes, direct_out=out_d, direct_lse_out=lse_d,
                           **kw)
    out_c = torch.empty_like(out_d)
    lse_c = torch.empty_like(lse_d)
    pkv.pkv_combine(workspace=ws, workspace_bytes=nbytes, num_partials=kw["num_partials"],
                    req_tile_base=kw["req_tile_base"], batch=inp.batch, q_len=inp.q_len,
                    num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                    out=out_c, lse_out=lse_c)
    torch.cuda.synchronize()
    single = inp.seq_lens <= kw["tile_tokens"]
    bd = out_d.view(torch.int16).cpu().numpy()
    bc = out_c.view(torch.int16).cpu().numpy()
    ld, lc = lse_d.cpu().numpy(), lse_c.cpu().numpy()
    log("  T=%d: %d of %d requests single-tile" % (kw["tile_tokens"], int(single.sum()), inp.batch))
    assert single.any()
    assert np.array_equal(bd[single], bc[single]) and np.array_equal(ld[single], lc[single])
    assert (out_d.float().cpu().numpy()[~single] == 7.0).all() and (ld[~single] == 7.0).all()


def test_empty_batch_is_a_no_op():
    import torch
    inp = synth.make_inputs(cfg(), seed=0, seq_lens=[5])
    runner = make_runner(inp)
    dev = device_inputs(inp)
    out = runner(dev["q"][:0], dev["k"], dev["v"], dev["bt"][:0], np.zeros(0, np.int32), inp.scale)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 1, 8, 128)
