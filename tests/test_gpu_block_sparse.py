"""Block-sparse decode on an MI355X against the fp64 oracle: the device compaction
bit for bit, whole steps (host and device plan, bf16 and fp8 KV, draft tokens) to the
decode tolerances, masked pages never read, and the full mixed and fp8 workloads
with every (request, kv head) group against the oracle."""

import numpy as np
import pytest

import synth
from tests.gpu_util import device_inputs, log
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def cfg(**kw):
    base = dict(name="sparse", batch=0, seq_lens=(1,), q_len=1, num_q_heads=8, num_kv_heads=2,
                head_dim=128, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def run_sparse(inp, mask, T=0, W=0, device_plan=False, dev=None):
    """One block-sparse step; returns (out float32, lse, out bf16 bits)."""
    import torch
    import paged_kv_gqa_amd as pkv
    dev = dev or device_inputs(inp)
    r = pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                        head_dim=inp.head_dim, page_size=inp.page_size, kv_format=inp.kv_format,
                        q_len=inp.q_len, tile_tokens=T, num_workers=W, device_plan=device_plan)
    mask_d = torch.from_numpy(mask).cuda()
    lse = torch.empty((inp.batch, inp.q_len, inp.num_q_heads), dtype=torch.float32, device="cuda")
    out = r(dev["q"], dev["k"], dev["v"], dev["bt"], inp.seq_lens, inp.scale, k_scale=dev["ks"],
            v_scale=dev["vs"], seq_lens=dev["sl"], lse_out=lse, block_mask=mask_d, block_mask_h=mask)
    torch.cuda.synchronize()
    if device_plan:
        assert r.plan_info()["status"] == 0
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.float().cpu().numpy(), lse.cpu().numpy(), bits


def check_sparse(inp, mask, out, lse, pairs=None, tag=""):
    check(inp, out, lse, pairs=pairs, tag=tag, block_mask=mask)


@pytest.mark.parametrize("q_len,P", [(1, 16), (4, 16), (2, 64)])
def test_compaction_is_exact(q_len, P):
    import torch
    import paged_kv_gqa_amd as pkv
    c = cfg(q_len=q_len, page_size=P, num_kv_heads=4)
    sl = [q_len, 15, 16, 17, 18, 100, 333, 1500]
    inp = synth.make_inputs(c, seed=2, slack_pages=4, seq_lens=[max(x, q_len) for x in sl])
    dev = device_inputs(inp)
    Hkv, B, S = 4, inp.batch, inp.block_table.shape[1]
    for keep in (0.0, 0.4, 1.0):
        mask = synth.make_block_mask(inp, keep, seed=3)
        bt_out = torch.full((B * Hkv, S), -7, dtype=torch.int32, device="cuda")
        sl_out = torch.full((B * Hkv,), -7, dtype=torch.int32, device="cuda")
        pkv.pkv_block_sparse_compact(block_table=dev["bt"], seq_lens=dev["sl"],
                                     block_mask=torch.from_numpy(mask).cuda(), batch=B, num_kv_heads=Hkv,
                                     q_len=q_len, page_size=P, bt_stride=S, mask_stride=S,
                                     num_pages=inp.num_pages, bt_out=bt_out, seq_lens_out=sl_out)
        torch.cuda.synchronize()
        got_bt, got_sl = bt_out.cpu().numpy(), sl_out.cpu().numpy()
        att = synth.attended_pages(inp, mask)
        for b in range(B):
            L = int(inp.seq_lens[b])
            for g in range(Hkv):
                v = b * Hkv + g
                pages = att[b][g]
                want = [int(inp.block_table[b, p]) * Hkv + g for p in pages]
                assert got_bt[v, :len(pages)].tolist() == want, (b, g, keep)
                assert (got_bt[v, len(pages):] == -7).all()
                assert got_sl[v] == sum(min(P, L - p * P) for p in pages)


SMALL = [
    dict(id="g4_p16_keep30", c=cfg(), keep=0.3, T=64, W=7),
    dict(id="g4_p16_keep0", c=cfg(), keep=0.0, T=0, W=0),
    dict(id="g4_p16_keep100", c=cfg(), keep=1.0, T=32, W=5),
    dict(id="spec4_g4_keep50", c=cfg(q_len=4), keep=0.5, T=48, W=3),
    dict(id="g1_d64_p32_keep40", c=cfg(num_q_heads=4, num_kv_heads=4, head_dim=64, page_size=32),
         keep=0.4, T=0, W=0),
    dict(id="g8_p64_keep25", c=cfg(num_q_heads=16, page_size=64), keep=0.25, T=128, W=9),
    dict(id="fp8_spec2_keep50", c=cfg(kv_format="fp8", page_size=64, q_len=2), keep=0.5, T=0, W=0),
    dict(id="fp8_spec4_g4_keep30", c=cfg(kv_format="fp8", page_size=64, q_len=4), keep=0.3, T=64, W=11),
    dict(id="p48_d64_spec2_keep40", c=cfg(page_size=48, head_dim=64, q_len=2, num_q_heads=16),
         keep=0.4, T=96, W=5),
    dict(id="fp8_d64_spec4_keep60", c=cfg(kv_format="fp8", page_size=64, head_dim=64, q_len=4),
         keep=0.6, T=0, W=0),
    dict(id="fp8_p16_spec2_keep40", c=cfg(kv_format="fp8", page_size=16, q_len=2), keep=0.4, T=64, W=5),
    dict(id="fp8_p32_spec4_keep50", c=cfg(kv_format="fp8", page_size=32, q_len=4), keep=0.5, T=0, W=0),
]
LENS = [1, 16, 17, 63, 64, 65, 200, 777, 1500, 3000]


@pytest.mark.parametrize("device_plan", [False, True])
@pytest.mark.parametrize("case", SMALL, ids=[c["id"] for c in SMALL])
def test_small_cases_match_oracle(case, device_plan):
    c = case["c"]
    inp = synth.make_inputs(c, seed=21, poison=True, slack_pages=3,
                            seq_lens=[max(x, c["q_len"]) for x in LENS])
    mask = synth.make_block_mask(inp, case["keep"], seed=22)
    log("sparse case %s device_plan=%s" % (case["id"], device_plan))
    out, lse, _ = run_sparse(inp, mask, case["T"], case["W"], device_plan=device_plan)
    check_sparse(inp, mask, out, lse, tag=case["id"])


def random_case(seed):
    """A random block-sparse batch from ``default_rng(seed)``: shape as in the random
    decode cases, a keep fraction, a fixed or automatic tile, workers, host or device
    plan."""
    rng = np.random.default_rng(4000 + seed)
    Tq = int(rng.integers(1, 5))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16, 32) if g * Tq <= 64]))
    Hkv = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([16, 32, 48, 64]))
    fmt = str(rng.choice(["bf16", "fp8"]))
    c = cfg(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=int(rng.choice([64, 128])),
            page_size=P, kv_format=fmt, q_len=Tq)
    sl = [int(x) for x in rng.integers(Tq, 2500, int(rng.integers(1, 9)))]
    quantum = P if fmt == "bf16" else P * 64 // int(np.gcd(P, 64))
    T = 0 if rng.random() < 0.4 else quantum * int(rng.integers(1, 6))
    return (c, sl, float(rng.choice([0.1, 0.3, 0.6, 1.0])), T, int(rng.integers(1, 12)),
            bool(rng.random() < 0.5))


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_match_oracle(seed):
    c, sl, keep, T, W, device_plan = random_case(seed)
    inp = synth.make_inputs(c, seed=70 + seed, poison=True, slack_pages=2, seq_lens=sl)
    mask = synth.make_block_mask(inp, keep, seed=80 + seed)
    tag = "random %d: B=%d Tq=%d Hq=%d Hkv=%d D=%d P=%d %s keep=%.1f T=%d W=%d device_plan=%s" % (
        seed, inp.batch, inp.q_len, inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
        inp.kv_format, keep, T, W, device_plan)
    log(tag)
    out, lse, _ = run_sparse(inp, mask, T=T, W=W, device_plan=device_plan)
    check_sparse(inp, mask, out, lse, tag=tag)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_host_and_device_plans_agree_bitwise(fmt):
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2, num_q_heads=16, num_kv_heads=4)
    inp = synth.make_inputs(c, seed=23, seq_lens=[2, 100, 1000, 2500, 4000, 64])
    mask = synth.make_block_mask(inp, 0.35, seed=24)
    dev = device_inputs(inp)
    _, l1, b1 = run_sparse(inp, mask, dev=dev)
    _, l2, b2 = run_sparse(inp, mask, device_plan=True, dev=dev)
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_masked_pages_are_never_read(fmt):
    """NaN in every page the mask leaves out (and in the usual unread places) changes
    nothing, bit for bit."""
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=3, num_kv_heads=4,
            num_q_heads=16)
    lens = [3, 90, 700, 2049, 3000]
    clean = synth.make_inputs(c, seed=25, seq_lens=lens)
    dirty = synth.make_inputs(c, seed=25, seq_lens=lens)
    mask = synth.make_block_mask(clean, 0.3, seed=26)
    synth.apply_poison(dirty)
    att = synth.attended_pages(dirty, mask)
    nan = synth.BF16_NAN if fmt == "bf16" else synth.FP8_NAN
    P = dirty.page_size
    for b in range(dirty.batch):
        n = (int(dirty.seq_lens[b]) + P - 1) // P
        for g in range(dirty.num_kv_heads):
            for p in set(range(n)) - set(att[b][g]):
                phys = dirty.block_table[b, p]
                dirty.k_cache[phys, g] = nan
                dirty.v_cache[phys, g] = nan
    _, l1, b1 = run_sparse(clean, mask)
    _, l2, b2 = run_sparse(dirty, mask)
    assert np.isfinite(l2).all()
    assert np.array_equal(b1, b2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name,keep", [("mixed", 0.25), ("fp8_spec", 0.5)])
def test_full_size_sparse(name, keep):
    import torch
    log("full-size sparse %s keep %.2f: generating inputs" % (name, keep))
    inp = synth.make_inputs(synth.ALL[name], seed=0)
    mask = synth.make_block_mask(inp, keep, seed=1)
    out, lse, _ = run_sparse(inp, mask)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    log("full-size sparse %s: oracle over all %d groups" % (name, inp.batch * inp.num_kv_heads))
    check_sparse(inp, mask, out, lse, tag="%s keep %.2f" % (name, keep))
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_million_token_request(fmt):
    """A 1 000 003-token request with about 40 % of its pages attended, beside a short
    one, two kv heads (masks differ per head), two draft tokens: the compaction walks
    ~62 500 mask bytes per row (bf16 pages of 16); host and device plans give the same
    bits, every row checked against the oracle."""
    import torch
    c = cfg(q_len=2, num_q_heads=4, num_kv_heads=2, kv_format=fmt, page_size=64 if fmt == "fp8" else 16)
    inp = synth.make_inputs(c, seed=44, seq_lens=[1_000_003, 300])
    mask = synth.make_block_mask(inp, 0.4, seed=45)
    dev = device_inputs(inp)
    log("block-sparse 1M-token request (%s): %d pages, %d mask bytes per row" % (
        fmt, inp.k_cache.shape[0], mask.shape[-1]))
    out, lse, bits = run_sparse(inp, mask, dev=dev)
    check_sparse(inp, mask, out, lse, tag="sparse 1M %s" % fmt)
    _, lse_d, bits_d = run_sparse(inp, mask, device_plan=True, dev=dev)
    assert np.array_equal(bits, bits_d) and np.array_equal(lse, lse_d)
    del dev
    torch.cuda.empty_cache()


def test_graph_replay_with_new_masks_and_lengths():
    """Compaction + device plan + decode + combine captured once, replayed with new
    device masks and lengths; every replay equals an eager host-planned block-sparse
    step bit for bit."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = cfg(q_len=2, num_q_heads=16, num_kv_heads=4)
    B = 16
    inp = synth.make_inputs(dict(c, batch=B), seed=46, seq_lens=np.full(B, 5000, np.int32))
    dev = device_inputs(inp)
    rng = np.random.default_rng(47)
    r = pkv.PagedDecode(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16, q_len=2,
                        device_plan=True)
    static_sl = dev["sl"].clone()
    static_mask = torch.from_numpy(synth.make_block_mask(inp, 0.5, seed=48)).cuda()
    out = torch.empty((B, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 2, 16), dtype=torch.float32, device="cuda")

    def step():
        r(dev["q"], dev["k"], dev["v"], dev["bt"], None, inp.scale, seq_lens=static_sl, out=out,
          lse_out=lse, block_mask=static_mask)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # buffers and workspace exist before the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    host = pkv.PagedDecode(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16, q_len=2)
    for rep in range(4):
        new_sl = np.maximum(rng.integers(2, 5001, B), 2).astype(np.int32)
        new_mask = synth.make_block_mask(inp, [0.1, 0.5, 0.9, 0.3][rep], seed=49 + rep)
        static_sl.copy_(torch.from_numpy(new_sl))
        static_mask.copy_(torch.from_numpy(new_mask))
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()
        ref_lse = torch.empty_like(lse)
        ref = host(dev["q"], dev["k"], dev["v"], dev["bt"], new_sl, inp.scale,
                   seq_lens=torch.from_numpy(new_sl).cuda(), lse_out=ref_lse,
                   block_mask=torch.from_numpy(new_mask).cuda(), block_mask_h=new_mask)
        torch.cuda.synchronize()
        info = r.plan_info()
        log("  replay %d: %s" % (rep, info))
        assert info["status"] == 0
        assert np.array_equal(got, ref.view(torch.int16).cpu().numpy()), rep
        assert np.array_equal(got_lse, ref_lse.cpu().numpy()), rep
