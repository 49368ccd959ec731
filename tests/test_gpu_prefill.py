"""Variable-length causal prefill on an MI355X against the fp64 prefill oracle.

Small batches are compared whole (every row, every head); the full-size workloads on
sampled rows (first and last tokens, tile and block boundaries, random tokens) of
sampled (request, kv head) pairs. Tolerances are the decode contract's: max |gpu -
oracle| <= 1e-2 on the bf16 output for BF16 KV, 3e-2 for FP8 KV (or 0.6 bf16 ulp of the
reference where that is larger), relative L2 <= 1e-2, |lse - lse_ref| <= 1e-3.

Properties that hold at any size: the rows of a chunk after a prefix match the same rows
of the whole prompt, and the order of the work items changes nothing (bit for bit).
"""

import numpy as np
import pytest

import synth
from oracle.prefill import prefill_attention
from tests.gpu_util import device_inputs, log, max_abs, pages_past_two_gib, rel_l2
from tests.test_gpu_parity import LSE_TOL, REL_TOL, TOL, excess

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def cfg(**kw):
    base = dict(name="prefill", batch=0, q_lens=("const", 1), prefix=("const", 0), num_q_heads=8,
                num_kv_heads=2, head_dim=128, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def device_prefill(p):
    import torch
    dev = device_inputs(p.cache)
    dev["pq"] = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    dev["cu"] = torch.from_numpy(p.cu_q).cuda()
    dev["kl"] = torch.from_numpy(p.cache.seq_lens).cuda()
    return dev


def run_prefill(p, dev=None, items=None, with_lse=True):
    """(out float32 [total, Hq, D], lse float32 [total, Hq] or None, out bf16 bits)."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = p.cache
    dev = dev or device_prefill(p)
    log("  prefill B=%d total=%d Hq=%d Hkv=%d D=%d P=%d %s" % (
        p.batch, int(p.cu_q[-1]), c.num_q_heads, c.num_kv_heads, c.head_dim, c.page_size, c.kv_format))
    runner = pkv.PagedPrefill(num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
                              head_dim=c.head_dim, page_size=c.page_size, kv_format=c.kv_format)
    total = int(p.cu_q[-1])
    lse = torch.full((total, c.num_q_heads), float("nan"), device="cuda") if with_lse else None
    out = torch.full_like(dev["pq"], float("nan"))
    if items is not None:
        items = torch.from_numpy(np.ascontiguousarray(items)).cuda()
    runner(dev["pq"], dev["cu"], dev["kl"], dev["bt"], p.q_lens, c.seq_lens, c.scale,
           k_cache=dev["k"], v_cache=dev["v"], k_scale=dev["ks"], v_scale=dev["vs"], out=out,
           lse=lse, items=items)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.float().cpu().numpy(), None if lse is None else lse.cpu().numpy(), bits


def compare(p, out, lse, ref_out, ref_lse, tag):
    sel = ~np.isnan(ref_lse)                                   # rows x heads the oracle computed
    o, ro = out[sel], ref_out[sel]
    assert np.isfinite(o).all(), tag
    ea, er = max_abs(o, ro), rel_l2(o, ro)
    el = max_abs(lse[sel], ref_lse[sel]) if lse is not None else 0.0
    log("  %s: %d rows, max_abs %.3e rel_l2 %.3e lse %.3e" % (tag, int(sel.sum()), ea, er, el))
    assert excess(o, ro, TOL[p.cache.kv_format]) <= 0, tag
    assert er <= REL_TOL, tag
    if lse is not None:
        assert np.isfinite(lse[sel]).all() and el <= LSE_TOL, tag


SMALL = [
    dict(id="g4_d128_p16_noprefix", c=cfg(), q=[1, 7, 63, 64, 65, 130], pre=[0] * 6),
    dict(id="g4_d128_p16_prefix", c=cfg(), q=[5, 33, 64, 100], pre=[11, 0, 70, 300]),
    dict(id="g1_d64_p32", c=cfg(num_q_heads=2, num_kv_heads=2, head_dim=64, page_size=32),
         q=[50, 3, 129], pre=[0, 100, 31]),
    dict(id="g2_d128_p16", c=cfg(num_q_heads=4, num_kv_heads=2), q=[31, 32, 33, 97], pre=[1, 2, 3, 200]),
    dict(id="g8_d64_p16", c=cfg(num_q_heads=16, num_kv_heads=2, head_dim=64), q=[20, 90], pre=[3, 0]),
    dict(id="g4_d64_p48", c=cfg(head_dim=64, page_size=48), q=[200, 17], pre=[49, 0]),
    dict(id="g12_d128_p16", c=cfg(num_q_heads=12, num_kv_heads=1), q=[77], pre=[40]),
    dict(id="fp8_g4_d128", c=cfg(kv_format="fp8", page_size=64), q=[70, 5, 128], pre=[0, 64, 60]),
    dict(id="fp8_g2_d64", c=cfg(kv_format="fp8", page_size=64, head_dim=64, num_q_heads=4),
         q=[1, 64, 65, 190], pre=[0, 1, 63, 129]),
    dict(id="fp8_g1_d128", c=cfg(kv_format="fp8", page_size=64, num_q_heads=2), q=[33, 300],
         pre=[500, 0]),
    dict(id="fp8_g4_d128_p16", c=cfg(kv_format="fp8", page_size=16), q=[70, 5, 128], pre=[0, 17, 60]),
    dict(id="fp8_g2_d64_p48", c=cfg(kv_format="fp8", page_size=48, head_dim=64, num_q_heads=4),
         q=[1, 47, 49, 190], pre=[0, 1, 95, 129]),
    dict(id="fp8_g8_d128_p32", c=cfg(kv_format="fp8", page_size=32, num_q_heads=8), q=[100, 33],
         pre=[31, 300]),
    # Four-head groups at D = 64: each of the 512 threads widens one 4-byte unit of a block.
    dict(id="fp8_g4_d64_p16", c=cfg(kv_format="fp8", page_size=16, head_dim=64), q=[3, 64, 97, 1],
         pre=[0, 33, 15, 95]),
]


@pytest.mark.parametrize("case", SMALL, ids=[c["id"] for c in SMALL])
def test_small_batches_match_the_oracle(case):
    p = synth.make_prefill_inputs(case["c"], seed=11, q_lens=case["q"], prefix=case["pre"],
                                  poison=True, slack_pages=3)
    out, lse, _ = run_prefill(p)
    ref_out, ref_lse = prefill_attention(p)
    compare(p, out, lse, ref_out, ref_lse, case["id"])


def random_case(seed):
    """A small random prefill batch: head group, kv heads, head dim, page size, format,
    query lengths and prefixes drawn from ``default_rng(seed)``."""
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([1, 2, 4, 8, 12]))  # the group sizes prefill supports
    Hkv = int(rng.choice([1, 2]))
    fmt = str(rng.choice(["bf16", "fp8"]))
    c = cfg(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=int(rng.choice([64, 128])),
            page_size=int(rng.choice([16, 32, 48, 64])), kv_format=fmt)
    B = int(rng.integers(1, 5))
    q = [int(x) for x in rng.integers(1, 200, B)]
    pre = [int(x) for x in rng.integers(0, 300, B)]
    return c, q, pre


@pytest.mark.parametrize("seed", range(12))
def test_random_small_batches_match_the_oracle(seed):
    """Random shapes: tiles of 1-4 blocks and longer, every head-group width (one, two or
    four heads per item), both formats, pages of 16-64 tokens, against the oracle."""
    c, q, pre = random_case(seed)
    p = synth.make_prefill_inputs(c, seed=30 + seed, q_lens=q, prefix=pre, poison=True,
                                  slack_pages=2)
    out, lse, _ = run_prefill(p)
    ref_out, ref_lse = prefill_attention(p)
    compare(p, out, lse, ref_out, ref_lse, "random %d: %s q=%s pre=%s" % (
        seed, {k: c[k] for k in ("num_q_heads", "num_kv_heads", "head_dim", "page_size",
                                 "kv_format")}, q, pre))


def test_without_lse_the_output_is_the_same():
    p = synth.make_prefill_inputs(cfg(), seed=12, q_lens=[70, 9], prefix=[5, 60])
    dev = device_prefill(p)
    _, _, a = run_prefill(p, dev=dev)
    _, _, b = run_prefill(p, dev=dev, with_lse=False)
    assert np.array_equal(a, b)


def test_item_order_changes_nothing():
    import paged_kv_gqa_amd as pkv
    p = synth.make_prefill_inputs(cfg(kv_format="fp8", page_size=64), seed=13, q_lens=[150, 64, 3],
                                  prefix=[10, 0, 200])
    c = p.cache
    dev = device_prefill(p)
    _, l1, a = run_prefill(p, dev=dev)
    items = pkv.pkv_prefill_plan(p.q_lens, c.seq_lens, c.num_q_heads, c.num_kv_heads)
    perm = np.random.default_rng(0).permutation(len(items))
    _, l2, b = run_prefill(p, dev=dev, items=items[perm])
    assert np.array_equal(a, b) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_chunk_rows_match_whole_prompt_rows(fmt):
    """A chunk of 100 tokens after a 157-token prefix against the whole 257-token prompt
    over the same cache: the GPU gives the same rows to the parity tolerance (the
    kernel's rescaling and low-part decisions depend on which rows share a wave, so the
    bits may differ), and both match the oracle."""
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16)
    chunk = synth.make_prefill_inputs(c, seed=14, q_lens=[100], prefix=[157])
    whole = synth.make_prefill_inputs(c, seed=14, q_lens=[100], prefix=[157])
    rng = np.random.default_rng(15)
    head = synth.f32_to_bf16_bits(rng.standard_normal((157,) + chunk.q.shape[1:], dtype=np.float32))
    whole.q = np.concatenate([head, chunk.q])
    whole.q_lens = np.array([257], np.int32)
    whole.cu_q = np.array([0, 257], np.int32)
    o1, l1, _ = run_prefill(chunk)
    o2, l2, _ = run_prefill(whole)
    assert excess(o1, o2[157:].astype(np.float64), TOL[fmt]) <= 0
    assert rel_l2(o1, o2[157:]) <= REL_TOL and max_abs(l1, l2[157:]) <= LSE_TOL
    ref_out, ref_lse = prefill_attention(chunk)
    compare(chunk, o1, l1, ref_out, ref_lse, "chunk")


def sample_rows(p, rng, per_request=12):
    rows = {}
    for b in range(p.batch):
        n = int(p.q_lens[b])
        cand = {0, n - 1, min(63, n - 1), min(64, n - 1), min(31, n - 1), n // 2}
        cand.update(int(x) for x in rng.integers(0, n, per_request))
        rows[b] = sorted(cand)
    return rows


@pytest.mark.parametrize("name", ["prefill_varlen", "prefill_chunk_fp8", "prefill_long"])
def test_full_size_sampled_rows(name):
    w = synth.ALL_PREFILL[name]
    p = synth.make_prefill_inputs(w, seed=0)
    out, lse, _ = run_prefill(p)
    rng = np.random.default_rng(1)
    Hkv = p.cache.num_kv_heads
    pairs = [(b, int(g)) for b in range(p.batch) for g in rng.choice(Hkv, 2, replace=False)]
    ref_out, ref_lse = prefill_attention(p, pairs=pairs, rows=sample_rows(p, rng))
    compare(p, out, lse, ref_out, ref_lse, name)
    assert np.isfinite(out).all() and np.isfinite(lse).all()     # every row of every head written


def test_empty_requests_are_skipped():
    """Requests with no query tokens (a prefix only) sit between others; an all-empty
    batch plans no work and launches nothing."""
    p = synth.make_prefill_inputs(cfg(), seed=21, q_lens=[0, 5, 0, 70], prefix=[9, 3, 40, 0],
                                  poison=True, slack_pages=2)
    out, lse, _ = run_prefill(p)
    ref_out, ref_lse = prefill_attention(p)
    compare(p, out, lse, ref_out, ref_lse, "empty_requests")
    empty = synth.make_prefill_inputs(cfg(), seed=22, q_lens=[0, 0], prefix=[4, 8])
    out, lse, _ = run_prefill(empty)
    assert out.shape[0] == 0 and lse.shape[0] == 0


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_negative_and_zero_scale(scale, fmt):
    """A negative softmax scale is taken exactly (Q's sign flipped; with FP8 K, before
    the query is split into its two e4m3 terms); a zero scale gives the mean of the
    visible V rows."""
    c = cfg() if fmt == "bf16" else cfg(kv_format="fp8", page_size=64)
    p = synth.make_prefill_inputs(c, seed=23, q_lens=[40, 9], prefix=[30, 0])
    p.cache.scale = np.float32(scale)
    out, lse, _ = run_prefill(p)
    ref_out, ref_lse = prefill_attention(p)
    compare(p, out, lse, ref_out, ref_lse, "scale_%g_%s" % (scale, fmt))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_query_rows_of_any_magnitude(fmt):
    """Query rows scaled by powers of two from 2^-24 (near-uniform weights) to 2^5 (sharp
    softmax, the running maximum raised often), and all-zero rows: with FP8 K each row
    enters the FP8 product as two e4m3 terms under its own power of two."""
    c = cfg() if fmt == "bf16" else cfg(kv_format="fp8", page_size=64)
    p = synth.make_prefill_inputs(c, seed=31, q_lens=[70, 129, 3], prefix=[20, 0, 250])
    q = (p.q.astype(np.uint32) << np.uint32(16)).view(np.float32)  # [tokens, Hq, D]
    rows = np.arange(q.shape[0] * q.shape[1]).reshape(q.shape[0], q.shape[1])
    factor = 2.0 ** np.array([-24.0, -8.0, 0.0, 3.0, 5.0])[rows % 5]
    factor[rows % 7 == 6] = 0.0
    p.q = synth.gen.f32_to_bf16_bits(q * factor[:, :, None].astype(np.float32))
    out, lse, _ = run_prefill(p)
    ref_out, ref_lse = prefill_attention(p)
    compare(p, out, lse, ref_out, ref_lse, "q_magnitudes_%s" % fmt)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_pages_past_two_gib(fmt):
    """The prompts' pages moved past 2^31 bytes into a ~2.2 GB cache tensor (the rest
    NaN): bit-identical output and lse."""
    import torch
    p = synth.make_prefill_inputs(cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16), seed=24,
                                  q_lens=[70, 130], prefix=[30, 200])
    dev = device_prefill(p)
    o1, l1, a = run_prefill(p, dev=dev)
    moved, base, nbytes = pages_past_two_gib(p.cache, dev)
    log("  prefill pages past 2 GiB (%s): first used page %d" % (fmt, base))
    o2, l2, b = run_prefill(p, dev=moved)
    assert np.array_equal(a, b) and np.array_equal(l1, l2)
    del moved, dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_chunk_after_million_token_prefix(fmt):
    """A 2048-token chunk after a 1 000 000-token prefix, beside a short prompt: query
    positions past 2^20, each tile walking ~31 300 key blocks through ~62 600 block-table
    entries (bf16 pages of 16); sampled rows of both requests against the oracle."""
    import torch
    p = synth.make_prefill_inputs(cfg(num_q_heads=4, num_kv_heads=1, kv_format=fmt,
                                      page_size=64 if fmt == "fp8" else 16),
                                  seed=25, q_lens=[2048, 50], prefix=[1_000_000, 3])
    log("  chunk after a 1M-token prefix (%s): %d pages" % (fmt, p.cache.k_cache.shape[0]))
    out, lse, _ = run_prefill(p)
    rows = sample_rows(p, np.random.default_rng(3), per_request=6)
    ref_out, ref_lse = prefill_attention(p, pairs=[(0, 0), (1, 0)], rows=rows)
    compare(p, out, lse, ref_out, ref_lse, "1M prefix %s" % fmt)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    torch.cuda.empty_cache()
