"""Fused KV append on an MI355X against the oracle, bit for bit: the whole cache and
scales after the append (bf16 and fp8, with and without rotation, 1-4 new tokens
across page boundaries, fresh pages, kept and raised fp8 scales), the rotated q,
repeated appends, e4m3fn special values, and a decode step over the appended cache
against the fp64 decode oracle."""

import numpy as np
import pytest

import synth
from oracle import append as OA
from tests.gpu_util import device_inputs, log, pages_past_two_gib, run_decode
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def cfg(**kw):
    base = dict(name="append", batch=0, seq_lens=(1,), q_len=1, num_q_heads=8, num_kv_heads=2,
                head_dim=128, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


def gpu_append(inp, dev, k_new, v_new, q, rope):
    """Run pkv_kv_append on the device copies in ``dev`` (updated in place); returns the
    rotated q bits (or None)."""
    import torch
    import paged_kv_gqa_amd as pkv
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    kn, vn = t(k_new), t(v_new)
    qd = t(q) if rope is not None else None
    q_out = torch.empty_like(qd) if qd is not None else None
    cos = sin = None
    if rope is not None:
        cos, sin = (torch.from_numpy(x).cuda() for x in rope)
    pkv.pkv_kv_append(k_new=kn, v_new=vn, k_cache=dev["k"], v_cache=dev["v"], block_table=dev["bt"],
                      seq_lens=dev["sl"], num_pages=dev["k"].shape[0], batch=inp.batch,
                      q_len=inp.q_len, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                      head_dim=inp.head_dim, page_size=inp.page_size, bt_stride=inp.block_table.shape[1],
                      kv_format=inp.kv_format, q=qd, q_out=q_out, rope_cos=cos, rope_sin=sin,
                      max_pos=0 if rope is None else rope[0].shape[0], k_scale=dev["ks"], v_scale=dev["vs"])
    torch.cuda.synchronize()
    return None if q_out is None else q_out.view(torch.int16).cpu().numpy().view(np.uint16)


def cache_bits(dev, inp):
    import torch
    if inp.kv_format == "bf16":
        f = lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16)
        return f(dev["k"]), f(dev["v"]), None, None
    return dev["k"].cpu().numpy(), dev["v"].cpu().numpy(), dev["ks"].cpu().numpy(), dev["vs"].cpu().numpy()


def oracle_append(inp, k_new, v_new, q, rope):
    cos, sin = rope if rope is not None else (None, None)
    q_out = OA.kv_append(inp.k_cache, inp.v_cache, inp.k_scale, inp.v_scale, inp.block_table,
                         inp.seq_lens, k_new, v_new, q=q, cos=cos, sin=sin, kv_format=inp.kv_format)
    return q_out


def assert_same(inp, dev, q_gpu, q_ref, tag):
    k, v, ks, vs = cache_bits(dev, inp)
    assert np.array_equal(k, inp.k_cache), tag + " k cache"
    assert np.array_equal(v, inp.v_cache), tag + " v cache"
    if ks is not None:
        for name, got, want in (("k_scale", ks, inp.k_scale), ("v_scale", vs, inp.v_scale)):
            bad = np.argwhere(got != want)
            for phys, g in bad[:8]:
                log("  %s %s[%d, %d]: gpu %r (%08x) oracle %r (%08x)" % (
                    tag, name, phys, g, float(got[phys, g]), got[phys, g:g + 1].view(np.uint32)[0],
                    float(want[phys, g]), want[phys, g:g + 1].view(np.uint32)[0]))
            assert len(bad) == 0, tag + " " + name
    if q_ref is not None:
        assert np.array_equal(q_gpu, q_ref), tag + " q"


CASES = [
    dict(id="bf16_p16_t1", c=cfg(), rope=False),
    dict(id="bf16_p16_t4_rope", c=cfg(q_len=4), rope=True),
    dict(id="bf16_p32_d64_t3_rope", c=cfg(q_len=3, page_size=32, head_dim=64, num_q_heads=8, num_kv_heads=8), rope=True),
    dict(id="bf16_p48_t4_rope", c=cfg(q_len=4, page_size=48), rope=True),
    dict(id="fp8_t1", c=cfg(kv_format="fp8", page_size=64), rope=False),
    dict(id="fp8_t2_rope", c=cfg(kv_format="fp8", page_size=64, q_len=2), rope=True),
    dict(id="fp8_t4_rope_g4", c=cfg(kv_format="fp8", page_size=64, q_len=4, num_q_heads=16, num_kv_heads=4), rope=True),
    dict(id="fp8_t3_d64", c=cfg(kv_format="fp8", page_size=64, q_len=3, head_dim=64), rope=False),
    dict(id="fp8_p16_t4_rope", c=cfg(kv_format="fp8", page_size=16, q_len=4), rope=True),
    dict(id="fp8_p32_t2", c=cfg(kv_format="fp8", page_size=32, q_len=2), rope=False),
    dict(id="fp8_p48_t3_rope_d64", c=cfg(kv_format="fp8", page_size=48, q_len=3, head_dim=64), rope=True),
]
# lengths hitting fresh pages (L - Tq on a page boundary), page-spanning new tokens,
# and pages with earlier tokens
LENS = [1, 4, 17, 63, 64, 65, 66, 67, 128, 130, 200, 1000]


@pytest.mark.parametrize("case", CASES, ids=[c["id"] for c in CASES])
def test_append_matches_oracle(case):
    c = case["c"]
    inp = synth.make_inputs(c, seed=31, slack_pages=3, seq_lens=[max(x, c["q_len"]) for x in LENS])
    # half the (request, kv head) groups far beyond their pages' range: fp8 scales rise
    scale = np.where(np.random.default_rng(32).random((inp.batch, inp.num_kv_heads)) < 0.5, 1.0, 3e3)
    k_new, v_new, q = synth.new_token_rows(inp, seed=33, scale=scale)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim) if case["rope"] else None
    dev = device_inputs(inp)
    log("append case %s" % case["id"])
    q_gpu = gpu_append(inp, dev, k_new, v_new, q, rope)
    q_ref = oracle_append(inp, k_new, v_new, q, rope)
    assert_same(inp, dev, q_gpu, q_ref, case["id"])


def random_case(seed):
    """A random append from ``default_rng(seed)``: format, page size, head dim, heads,
    new tokens (1-4), rotation or not, lengths, and which groups' new rows are scaled far
    beyond their pages' range."""
    rng = np.random.default_rng(3000 + seed)
    Tq = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    c = cfg(kv_format=str(rng.choice(["bf16", "fp8"])), page_size=int(rng.choice([16, 32, 48, 64])),
            head_dim=int(rng.choice([64, 128])), num_kv_heads=Hkv,
            num_q_heads=Hkv * int(rng.choice([1, 2, 4, 8])), q_len=Tq)
    lens = [int(x) for x in rng.integers(Tq, 700, int(rng.integers(1, 40)))]
    rope = bool(rng.random() < 0.6)
    far = rng.random((len(lens), Hkv)) < float(rng.choice([0.0, 0.3, 1.0]))
    return c, lens, rope, np.where(far, float(rng.choice([10.0, 3e3])), 1.0)


@pytest.mark.parametrize("seed", range(12))
def test_random_appends_match_oracle(seed):
    c, lens, rope_on, scale = random_case(seed)
    inp = synth.make_inputs(c, seed=50 + seed, slack_pages=2, seq_lens=lens)
    k_new, v_new, q = synth.new_token_rows(inp, seed=60 + seed, scale=scale)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim) if rope_on else None
    dev = device_inputs(inp)
    tag = "random %d: B=%d Tq=%d Hq=%d Hkv=%d D=%d P=%d %s rope=%s" % (
        seed, inp.batch, inp.q_len, inp.num_q_heads, inp.num_kv_heads, inp.head_dim, inp.page_size,
        inp.kv_format, rope_on)
    log(tag)
    q_gpu = gpu_append(inp, dev, k_new, v_new, q, rope)
    q_ref = oracle_append(inp, k_new, v_new, q, rope)
    assert_same(inp, dev, q_gpu, q_ref, tag)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_repeated_appends_match_oracle(fmt):
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2)
    lens = np.array([2, 61, 62, 63, 126, 300], np.int32)
    inp = synth.make_inputs(c, seed=34, slack_pages=4, seq_lens=lens + 2 * 8)   # room for 8 steps
    inp.seq_lens[:] = lens
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    dev = device_inputs(inp)
    import torch
    for step in range(8):
        dev["sl"].copy_(torch.from_numpy(inp.seq_lens))
        k_new, v_new, q = synth.new_token_rows(inp, seed=40 + step, scale=1.0 + 3 * step)
        q_gpu = gpu_append(inp, dev, k_new, v_new, q, rope)
        q_ref = oracle_append(inp, k_new, v_new, q, rope)
        assert_same(inp, dev, q_gpu, q_ref, "step %d" % step)
        inp.seq_lens += 2


def test_fp8_special_values_encode_exactly():
    """Rows whose largest value is 448 get scale 1 on a fresh page, so every other
    value is encoded as itself: grid midpoints (ties), subnormals, negative tiny values
    (-> 0x80), values between the last two grid points."""
    from oracle.formats import E4M3FN_TABLE
    c = cfg(kv_format="fp8", page_size=64, head_dim=128, num_kv_heads=1, num_q_heads=4)
    inp = synth.make_inputs(c, seed=35, slack_pages=2, seq_lens=[65, 129, 193])   # fresh pages
    grid = E4M3FN_TABLE[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2
    vals = np.concatenate([mids, -mids, [-2.0 ** -100, -0.0, 0.0, 2.0 ** -10, 3 * 2.0 ** -10, 440, 444]])
    rows = []
    for b in range(3):
        r = np.resize(vals[b * 127:], 128).astype(np.float32)
        r[0] = 448.0
        rows.append(r)
    x = np.stack(rows)[:, None, None, :]                       # [B, Tq=1, Hkv=1, D]
    kb = synth.f32_to_bf16_bits(x)
    assert np.array_equal(OA.bf16_bits_to_f64(kb).astype(np.float32), x.astype(np.float32))
    dev = device_inputs(inp)
    gpu_append(inp, dev, kb, kb, None, None)
    oracle_append(inp, kb, kb, None, None)
    assert_same(inp, dev, None, None, "special values")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_decode_after_append_matches_oracle(fmt):
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=4, num_q_heads=16,
            num_kv_heads=4)
    inp = synth.make_inputs(c, seed=36, slack_pages=2, seq_lens=[4, 70, 500, 2000, 3000])
    k_new, v_new, q = synth.new_token_rows(inp, seed=37)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    dev = device_inputs(inp)
    gpu_append(inp, dev, k_new, v_new, q, rope)
    q_rot = oracle_append(inp, k_new, v_new, q, rope)          # inp now holds the appended cache
    inp.q = q_rot
    import torch
    dev["q"] = torch.from_numpy(q_rot.view(np.int16)).view(torch.bfloat16).cuda()
    out, lse, _ = run_decode(inp, dev=dev)
    check(inp, out, lse, tag="append + decode " + fmt)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_pages_past_two_gib(fmt):
    """Appending into pages moved past 2^31 bytes of a ~2.2 GB cache tensor writes the
    same bits (codes and scales) as appending into the compact cache, and nothing
    before the moved pages."""
    import torch
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2)
    inp = synth.make_inputs(c, seed=35, slack_pages=2, seq_lens=[2, 17, 64, 65, 300, 1000])
    k_new, v_new, q = synth.new_token_rows(inp, seed=36)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    dev = device_inputs(inp)
    moved, base, _ = pages_past_two_gib(inp, dev)
    head = moved["k"][:base].view(torch.int16 if fmt == "bf16" else torch.uint8)[-4:].clone()
    q1 = gpu_append(inp, dev, k_new, v_new, q, rope)
    q2 = gpu_append(inp, moved, k_new, v_new, q, rope)
    assert np.array_equal(q1, q2)
    small = cache_bits(dev, inp)
    big = {name: moved[name][base:] for name in ("k", "v", "ks", "vs") if moved.get(name) is not None}
    for name, x in zip(("k", "v", "ks", "vs"), small):
        if x is None:
            continue
        y = big[name]
        y = y.view(torch.int16).cpu().numpy().view(np.uint16) if y.dtype == torch.bfloat16 else y.cpu().numpy()
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), name
    after = moved["k"][:base].view(torch.int16 if fmt == "bf16" else torch.uint8)[-4:]
    assert torch.equal(head, after)
    log("  append pages past 2 GiB (%s): first used page %d" % (fmt, base))
    del moved, dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_append_at_million_token_positions(fmt):
    """Four new tokens per request at positions past 10^6, both crossing a page boundary
    (999 999 | 1 000 000 and 1 048 575 | 1 048 576), rotated by tables of ~1.05M
    positions: the whole cache, the scales and the rotated q bit for bit."""
    import torch
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=4, num_q_heads=4,
            num_kv_heads=1)
    inp = synth.make_inputs(c, seed=36, seq_lens=[1_000_003, 1_048_578])
    k_new, v_new, q = synth.new_token_rows(inp, seed=37)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    dev = device_inputs(inp)
    log("append at 1M positions (%s): %d pages, tables of %d positions" % (
        fmt, inp.k_cache.shape[0], rope[0].shape[0]))
    q_gpu = gpu_append(inp, dev, k_new, v_new, q, rope)
    q_ref = oracle_append(inp, k_new, v_new, q, rope)
    assert_same(inp, dev, q_gpu, q_ref, "1M positions " + fmt)
    del dev
    torch.cuda.empty_cache()


def test_graph_captured_step_with_append():
    """A whole decode step with no host work - fused append (rotation, paged write) of
    the step's token, device plan, decode, combine - captured once in a HIP graph and
    replayed for four successive tokens with new rows and lengths; every replay's
    output, and the cache at the end, bit for bit those of the same steps run eagerly
    with host plans on a second copy of the cache."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = cfg(num_q_heads=16, num_kv_heads=4)
    lens = np.array([1, 15, 16, 17, 300, 1000, 2047], np.int32)
    inp = synth.make_inputs(c, seed=50, slack_pages=8, seq_lens=lens + 5)   # room for 5 tokens
    inp.seq_lens[:] = lens
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    cos, sin = (torch.from_numpy(x).cuda() for x in rope)
    dev_g, dev_e = device_inputs(inp), device_inputs(inp)
    kw = dict(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16)
    r_g, r_e = pkv.PagedDecode(device_plan=True, **kw), pkv.PagedDecode(**kw)
    as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    B = inp.batch
    kn, vn = (torch.empty((B, 1, 4, 128), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    qn = torch.empty((B, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    q_rot = torch.empty_like(qn)
    sl = dev_g["sl"]
    out = torch.empty((B, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, 16), dtype=torch.float32, device="cuda")

    def next_token(step):
        inp.seq_lens += 1
        k_h, v_h, q_h = synth.new_token_rows(inp, seed=60 + step)
        kn.copy_(as_bf16(k_h)); vn.copy_(as_bf16(v_h)); qn.copy_(as_bf16(q_h))
        sl.copy_(torch.from_numpy(inp.seq_lens))

    def graph_step():
        r_g.append(kn, vn, dev_g["k"], dev_g["v"], dev_g["bt"], sl, q=qn, q_out=q_rot,
                   rope_cos=cos, rope_sin=sin)
        r_g(q_rot, dev_g["k"], dev_g["v"], dev_g["bt"], None, inp.scale, seq_lens=sl, out=out,
            lse_out=lse)

    def eager_step():
        sl_e = torch.from_numpy(inp.seq_lens.copy()).cuda()
        q_e = torch.empty_like(qn)
        r_e.append(kn.clone(), vn.clone(), dev_e["k"], dev_e["v"], dev_e["bt"], sl_e, q=qn.clone(),
                   q_out=q_e, rope_cos=cos, rope_sin=sin)
        lse_e = torch.empty_like(lse)
        o = r_e(q_e, dev_e["k"], dev_e["v"], dev_e["bt"], inp.seq_lens.copy(), inp.scale,
                seq_lens=sl_e, lse_out=lse_e)
        return o, lse_e

    next_token(0)                   # first token: eager on both copies (allocates buffers)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        graph_step()
    torch.cuda.current_stream().wait_stream(s)
    eager_step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph_step()
    for step in range(1, 5):
        next_token(step)
        g.replay()
        torch.cuda.synchronize()
        got, got_lse = out.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()
        ref, ref_lse = eager_step()
        torch.cuda.synchronize()
        assert r_g.plan_info()["status"] == 0
        assert np.array_equal(got, ref.view(torch.int16).cpu().numpy()), step
        assert np.array_equal(got_lse, ref_lse.cpu().numpy()), step
        log("  token %d: replay equals the eager step" % step)
    for name in ("k", "v"):
        assert torch.equal(dev_g[name].view(torch.int16), dev_e[name].view(torch.int16)), name


@pytest.mark.parametrize("P", [16, 64])
def test_reappending_the_same_rows_matches_oracle(P):
    """The same new rows appended again at the same positions (as a benchmark loop does):
    where fl(a / s) lands just above 448 while fl(a / 448) == s, the rule raises the scale
    to its own value and re-encodes every earlier code to itself; the kernel skips that
    no-op and must still equal the oracle bit for bit, on every repeat."""
    import torch
    c = cfg(kv_format="fp8", page_size=P, q_len=4, num_q_heads=16, num_kv_heads=4)
    lens = [5, 6, 7, 30, 61, 62, 63, 100, 127, 200, 301, 777]
    inp = synth.make_inputs(c, seed=51, slack_pages=2, seq_lens=lens)
    k_new, v_new, q = synth.new_token_rows(inp, seed=52, scale=3.0)   # beyond the pages: scales rise
    dev = device_inputs(inp)
    equal_raises = 0
    for rep in range(4):
        dev["sl"].copy_(torch.from_numpy(inp.seq_lens))
        if rep > 0:  # count the pages whose scale the rule raises to the same value
            for b, L in enumerate(inp.seq_lens):
                first = int(L) - inp.q_len
                lp = first // P
                o0 = first - lp * P
                if o0 == 0:
                    continue
                phys = int(inp.block_table[b, lp])
                n = min(int(L), (lp + 1) * P) - first
                for g in range(inp.num_kv_heads):
                    for rows, sc in ((k_new, inp.k_scale), (v_new, inp.v_scale)):
                        vals = (rows[b, :n, g].astype(np.uint32) << 16).view(np.float32)
                        a = np.float32(np.max(np.abs(vals)))
                        s = np.float32(sc[phys, g])
                        if not (np.float32(a / s) <= np.float32(448.0)) and np.float32(a / np.float32(448.0)) == s:
                            equal_raises += 1
        gpu_append(inp, dev, k_new, v_new, None, None)
        oracle_append(inp, k_new, v_new, None, None)
        assert_same(inp, dev, None, None, "repeat %d" % rep)
    log("  P=%d: %d equal-scale raises over the repeats" % (P, equal_raises))
    assert equal_raises > 0


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_rope_tables_with_4_byte_alignment(fmt):
    """Rotation tables that are 4-byte but not 16-byte aligned (the contract's minimum):
    the kernel reads them element by element and must match the oracle bit for bit."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2, num_q_heads=8, num_kv_heads=2)
    inp = synth.make_inputs(c, seed=61, slack_pages=2, seq_lens=[2, 17, 64, 65, 300])
    k_new, v_new, q = synth.new_token_rows(inp, seed=62, scale=2.0)
    rope = synth.rope_tables(inp.block_table.shape[1] * inp.page_size, inp.head_dim)
    dev = device_inputs(inp)
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    tabs = []
    for x in rope:
        flat = torch.zeros(x.size + 1, dtype=torch.float32, device="cuda")
        flat[1:] = torch.from_numpy(x.reshape(-1)).cuda()
        tab = flat[1:].view(x.shape)
        assert tab.data_ptr() % 16 == 4
        tabs.append(tab)
    qd = t(q)
    q_out = torch.empty_like(qd)
    pkv.pkv_kv_append(k_new=t(k_new), v_new=t(v_new), k_cache=dev["k"], v_cache=dev["v"], block_table=dev["bt"],
                      seq_lens=dev["sl"], num_pages=dev["k"].shape[0], batch=inp.batch, q_len=inp.q_len,
                      num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim,
                      page_size=inp.page_size, bt_stride=inp.block_table.shape[1], kv_format=inp.kv_format,
                      q=qd, q_out=q_out, rope_cos=tabs[0], rope_sin=tabs[1], max_pos=rope[0].shape[0],
                      k_scale=dev["ks"], v_scale=dev["vs"])
    torch.cuda.synchronize()
    q_ref = oracle_append(inp, k_new, v_new, q, rope)
    assert_same(inp, dev, q_out.view(torch.int16).cpu().numpy().view(np.uint16), q_ref, "unaligned tables")
