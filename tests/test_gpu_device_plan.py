"""The device-built plan (pkv_plan_device) on an MI355X: bit for bit the reference
planner's work list (oracle.plan) for fixed and automatic tiles, the item-capacity
rule, errors reported on the device, and whole decode steps - eager and replayed
from a captured graph - against the host-planned step and the fp64 oracle."""

import numpy as np
import pytest

import synth
from oracle import plan as ref_plan
from tests.gpu_util import device_inputs, log, make_runner, run_decode

pytestmark = pytest.mark.gpu

SEQ, UNSUPPORTED, WORKSPACE = -6, -2, -4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def device_plan(seq_lens, q_len, Hq, Hkv, D, P, fmt, T, W, cap):
    """Run pkv_plan_device; returns (info, items [N,4], offsets, rtb) as numpy."""
    import torch
    import paged_kv_gqa_amd as pkv
    dev = torch.device("cuda", 0)
    B = len(seq_lens)
    i32 = dict(dtype=torch.int32, device=dev)
    sl = torch.tensor(np.asarray(seq_lens, np.int32), **i32)
    items = torch.full((max(cap, 1), 4), -7, **i32)       # -7: never written by a valid plan
    offs = torch.full((W + 1,), -7, **i32)
    rtb = torch.full((B + 1,), -7, **i32)
    info = torch.full((4,), -7, **i32)
    nscr = pkv.pkv_plan_device_scratch_bytes(B, Hkv, P, fmt, T, W, cap)
    scratch = torch.empty(nscr, dtype=torch.uint8, device=dev)
    pkv.pkv_plan_device(seq_lens=sl if B else None, batch=B, q_len=q_len, num_q_heads=Hq,
                        num_kv_heads=Hkv, head_dim=D, page_size=P, kv_format=fmt, tile_tokens=T,
                        num_workers=W, max_items=cap, items=items, worker_offsets=offs,
                        req_tile_base=rtb, info=info, scratch=scratch, scratch_bytes=nscr)
    torch.cuda.synchronize()
    info = info.cpu().numpy()
    N = max(int(info[2]), 0)
    return info, items.cpu().numpy()[:N], offs.cpu().numpy(), rtb.cpu().numpy()


def max_candidate_items(seq_lens, Hkv, fmt, P):
    q = ref_plan.tile_quantum(P, fmt)
    return Hkv * sum((int(L) + q - 1) // q for L in seq_lens)


def assert_matches_oracle(seq_lens, q_len, Hq, Hkv, D, P, fmt, T, W, cap, tag=""):
    info, items, offs, rtb = device_plan(seq_lens, q_len, Hq, Hkv, D, P, fmt, T, W, cap)
    ref = ref_plan.plan(seq_lens, q_len, Hq, Hkv, D, P, fmt, T, W, max_items=None if T else cap)
    N = len(ref["items"])
    counts = np.diff(ref["worker_offsets"])
    assert info[0] == 0, (tag, info)
    assert info[1] == ref["tile_tokens"], (tag, info, ref["tile_tokens"])
    assert info[2] == N and info[3] == (counts.max() if W else 0), (tag, info)
    assert np.array_equal(items, ref["items"]), tag
    assert np.array_equal(offs, ref["worker_offsets"]), tag
    assert np.array_equal(rtb, ref["req_tile_base"]), tag
    return int(info[1]), N


@pytest.mark.parametrize("name", list(synth.ALL))
@pytest.mark.parametrize("W", [100, 256, 512, 1024])   # 256: the default on MI355X
def test_workloads_match_oracle(name, W):
    c = synth.ALL[name]
    sl = synth.draw_seq_lens(c, np.random.default_rng(0))
    args = (c["q_len"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["page_size"], c["kv_format"])
    cap = max_candidate_items(sl, c["num_kv_heads"], c["kv_format"], c["page_size"])
    T, N = assert_matches_oracle(sl, *args, 0, W, cap, tag="%s auto W%d" % (name, W))
    log("  %s W=%d: auto T=%d N=%d" % (name, W, T, N))
    q = ref_plan.tile_quantum(c["page_size"], c["kv_format"])
    for Tf in (q, 4 * q, 3 * q):
        n_items = c["num_kv_heads"] * sum((int(L) + Tf - 1) // Tf for L in sl)
        assert_matches_oracle(sl, *args, Tf, W, n_items, tag="%s T%d W%d" % (name, Tf, W))


@pytest.mark.parametrize("B,W", [(300, 500), (600, 256), (1500, 512), (4096, 1024)])
def test_large_batches_match_oracle(B, W):
    """Request counts past one key per thread: 512-thread workgroups (W and B at most
    512), 1024-thread ones with the register sort of the request keys (B <= 1024), and
    with the LDS sort (B > 1024, up to the 4096 limit)."""
    rng = np.random.default_rng(B + W)
    sl = [int(x) for x in np.maximum(np.exp(rng.uniform(0, np.log(3000), B)).astype(int), 1)]
    Hkv = 2
    cap = max_candidate_items(sl, Hkv, "bf16", 16)
    T, N = assert_matches_oracle(sl, 1, 8, Hkv, 128, 16, "bf16", 0, W, cap, tag="B%d W%d auto" % (B, W))
    log("  B=%d W=%d: auto T=%d N=%d" % (B, W, T, N))
    n_items = Hkv * sum((L + 63) // 64 for L in sl)
    assert_matches_oracle(sl, 1, 8, Hkv, 128, 16, "bf16", 64, W, n_items, tag="B%d W%d T64" % (B, W))


def test_page_size_48_matches_oracle():
    """A page size that is not a power of two: quantum 48, candidates 48 .. 49152."""
    rng = np.random.default_rng(48)
    sl = [int(x) for x in rng.integers(1, 5000, 40)]
    cap = max_candidate_items(sl, 4, "bf16", 48)
    assert_matches_oracle(sl, 1, 16, 4, 128, 48, "bf16", 0, 333, cap, tag="P48 auto")
    n_items = 4 * sum((L + 143) // 144 for L in sl)
    assert_matches_oracle(sl, 1, 16, 4, 128, 48, "bf16", 144, 64, n_items, tag="P48 T144")


def test_random_shapes_match_oracle():
    rng = np.random.default_rng(2024)
    for case in range(150):
        B = int(rng.integers(0, 64))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4]))
        fmt = "fp8" if case % 5 == 4 else "bf16"
        P = int(rng.choice([16, 32, 48, 64]))
        q_len = int(rng.choice([1, 1, 2, 4])) if G * 4 <= 16 else 1
        W = int(rng.choice([1, 2, 7, 64, 333, 1024]))
        q = ref_plan.tile_quantum(P, fmt)
        kind = case % 3
        if kind == 0:
            sl = rng.integers(q_len, 2000, B)
        elif kind == 1:  # on and next to tile multiples
            sl = np.maximum(rng.integers(1, 6, B) * 256 + rng.integers(-1, 2, B), q_len)
        else:
            sl = np.maximum(np.exp(rng.uniform(0, np.log(4000), B)).astype(int), q_len)
        T = int(rng.choice([0, 0, q, 3 * q, 1024 // q * q or q]))
        if T:
            cap = Hkv * sum((int(L) + T - 1) // T for L in sl)
        else:  # between the largest candidate's items and the smallest's: may restrict
            lo = Hkv * sum((int(L) + 65535) // 65536 for L in sl)
            hi = max_candidate_items(sl, Hkv, fmt, P)
            cap = int(rng.integers(lo, hi + 1)) if hi > lo else hi
        assert_matches_oracle(list(sl), q_len, G * Hkv, Hkv, 128, P, fmt, T, W, cap,
                              tag="case %d B%d Hkv%d W%d T%d cap%d" % (case, B, Hkv, W, T, cap))


def test_capacity_restricts_the_automatic_tile():
    c = synth.MIXED
    sl = synth.draw_seq_lens(c, np.random.default_rng(0))
    args = (c["q_len"], c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["page_size"], c["kv_format"])
    T_free = ref_plan.auto_tile_tokens(sl, *args, 512)
    N_free = c["num_kv_heads"] * sum((int(L) + T_free - 1) // T_free for L in sl)
    T, N = assert_matches_oracle(sl, *args, 0, 512, N_free - 1, tag="restricted")
    assert T != T_free and N <= N_free - 1
    log("  mixed: free T=%d N=%d, capacity %d -> T=%d N=%d" % (T_free, N_free, N_free - 1, T, N))


def test_too_many_items_for_a_fixed_tile():
    # (ceil(100/16) + ceil(300/16)) * 2 kv heads = 52 items
    info, items, offs, rtb = device_plan([100, 300], 1, 8, 2, 128, 16, "bf16", 16, 64, 52)
    assert info[0] == 0 and info[2] == 52 and len(items) == 52
    info, _, offs, rtb = device_plan([100, 300], 1, 8, 2, 128, 16, "bf16", 16, 64, 51)
    assert info[0] == WORKSPACE and info[2] == 0
    assert (offs == 0).all() and (rtb == 0).all()


@pytest.mark.parametrize("sl,q_len", [([5, 0, 7], 1), ([5, 3, 7], 4), ([9, -1], 1)])
def test_short_sequences_are_reported(sl, q_len):
    for T in (0, 32):
        info, _, offs, rtb = device_plan(sl, q_len, 4, 1, 64, 16, "bf16", T, 8, 1000)
        assert info[0] == SEQ, info
        assert (offs == 0).all() and (rtb == 0).all()


def test_empty_batch():
    info, items, offs, rtb = device_plan([], 1, 8, 2, 128, 16, "bf16", 0, 64, 10)
    assert info[0] == 0 and info[2] == 0 and len(items) == 0
    assert (offs == 0).all() and list(rtb) == [0]


# ---------------------------------------------------------------------------------
# Whole decode steps


def run_both(inp, T=0, W=0):
    import torch
    dev = device_inputs(inp)
    host = run_decode(inp, T, W, dev=dev)
    import paged_kv_gqa_amd as pkv
    r = pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                        head_dim=inp.head_dim, page_size=inp.page_size, kv_format=inp.kv_format,
                        q_len=inp.q_len, tile_tokens=T, num_workers=W, device_plan=True)
    lse = torch.empty((inp.batch, inp.q_len, inp.num_q_heads), dtype=torch.float32, device="cuda")
    out = r(dev["q"], dev["k"], dev["v"], dev["bt"], None, inp.scale, k_scale=dev["ks"],
            v_scale=dev["vs"], seq_lens=dev["sl"], lse_out=lse)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return host, (out.float().cpu().numpy(), lse.cpu().numpy(), bits), r.plan_info()


@pytest.mark.parametrize("name", ["tiny", "llama8b", "mixed", "long", "fp8_spec"])
def test_step_equals_host_planned_step(name):
    inp = synth.make_inputs(synth.ALL[name], seed=0)
    host, devp, info = run_both(inp)
    log("  %s: device plan %s" % (name, info))
    assert info["status"] == 0
    assert np.array_equal(host[2], devp[2]) and np.array_equal(host[1], devp[1])


def test_step_matches_oracle_with_fixed_tile():
    from tests.test_gpu_parity import check
    for name, T, W in (("tiny", 16, 5), ("tiny", 0, 1)):
        inp = synth.make_inputs(synth.ALL[name], seed=3)
        _, (out, lse, _), info = run_both(inp, T, W)
        assert info["status"] == 0
        check(inp, out, lse, tag="%s T%d W%d" % (name, T, W))
    c = dict(synth.FP8_SPEC, batch=6, seq_lens=(4, 63, 64, 65, 700, 1500))
    inp = synth.make_inputs(c, seed=5)
    _, (out, lse, _), info = run_both(inp, 128, 7)
    check(inp, out, lse, tag="fp8 spec T128 W7")


def test_error_plan_gives_zeros():
    import torch
    inp = synth.make_inputs(dict(synth.TINY), seed=0)
    dev = device_inputs(inp)
    import paged_kv_gqa_amd as pkv
    r = pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                        head_dim=inp.head_dim, page_size=inp.page_size, q_len=1, device_plan=True)
    sl = dev["sl"].clone()
    sl[1] = 0
    lse = torch.empty((inp.batch, 1, inp.num_q_heads), dtype=torch.float32, device="cuda")
    out = r(dev["q"], dev["k"], dev["v"], dev["bt"], None, inp.scale, seq_lens=sl, lse_out=lse)
    torch.cuda.synchronize()
    assert r.plan_info()["status"] == SEQ
    assert (out.float() == 0).all().item() and torch.isinf(lse).all().item()


def test_graph_replay_with_new_lengths():
    """Plan + decode + combine captured once, replayed with new device seq_lens; every
    replay equals an eager host-planned step bit for bit."""
    import torch
    import paged_kv_gqa_amd as pkv
    c = dict(name="graph", batch=24, seq_lens=("loguniform", 64, 6000), q_len=2, num_q_heads=16,
             num_kv_heads=4, head_dim=128, page_size=16, kv_format="bf16")
    rng = np.random.default_rng(11)
    longest = np.full(24, 6000, np.int32)
    inp = synth.make_inputs(c, seed=11, seq_lens=longest)
    dev = device_inputs(inp)
    r = pkv.PagedDecode(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16, q_len=2,
                        device_plan=True)
    static_sl = dev["sl"].clone()
    out = torch.empty((24, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((24, 2, 16), dtype=torch.float32, device="cuda")

    def step():
        r(dev["q"], dev["k"], dev["v"], dev["bt"], None, inp.scale, seq_lens=static_sl, out=out,
          lse_out=lse)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                      # buffers and workspace exist before the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    host = make_runner(inp)
    for rep in range(4):
        new = np.maximum(np.exp(rng.uniform(np.log(2), np.log(6000), 24)).astype(np.int32), 2)
        static_sl.copy_(torch.from_numpy(new))
        g.replay()
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().copy()
        got_lse = lse.cpu().numpy().copy()
        ref_lse = torch.empty_like(lse)
        ref_out = host(dev["q"], dev["k"], dev["v"], dev["bt"], new, inp.scale,
                       seq_lens=torch.from_numpy(new).cuda(), lse_out=ref_lse)
        torch.cuda.synchronize()
        info = r.plan_info()
        log("  replay %d: %s" % (rep, info))
        assert info["status"] == 0
        assert np.array_equal(got, ref_out.view(torch.int16).cpu().numpy()), rep
        assert np.array_equal(got_lse, ref_lse.cpu().numpy()), rep
