"""PKV_VALIDATE: the synchronous checks of device-resident arguments (needs an MI355X).

With the variable set, valid steps give the same bits as without it, and a caller's
bad length, block-table entry or work list comes back as a pkv_status before any
kernel runs (the output buffers keep their NaN fill). Every bad input here still
points inside real memory - a "bad" page is a real page past a shortened num_pages,
a lengthened request reads block-table entries that hold real pages - so the tests
stay harmless even if a check failed to fire.
"""

import numpy as np
import pytest

import synth
from tests.gpu_util import device_inputs, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def cfg(**kw):
    base = dict(name="validate", batch=0, seq_lens=(1,), q_len=1, num_q_heads=8, num_kv_heads=2,
                head_dim=128, page_size=16, kv_format="bf16")
    base.update(kw)
    return base


SEQ = [1, 15, 16, 17, 33, 100, 257, 700]


def runner(inp, T=64, W=7, **kw):
    import paged_kv_gqa_amd as pkv
    return pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                           head_dim=inp.head_dim, page_size=inp.page_size, kv_format=inp.kv_format,
                           q_len=inp.q_len, tile_tokens=T, num_workers=W, **kw)


def decode(inp, dev, r=None, seq_lens_h=None, seq_lens=None, pages=None, **kw):
    """One step into NaN-filled buffers; `pages` shortens the cache views (num_pages)."""
    import torch
    r = r or runner(inp)
    out = torch.full((inp.batch, inp.q_len, inp.num_q_heads, inp.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    lse = torch.full((inp.batch, inp.q_len, inp.num_q_heads), float("nan"), device="cuda")
    n = pages or dev["k"].shape[0]
    ks = None if dev["ks"] is None else dev["ks"][:n]
    vs = None if dev["vs"] is None else dev["vs"][:n]
    r(dev["q"], dev["k"][:n], dev["v"][:n], dev["bt"], inp.seq_lens if seq_lens_h is None else seq_lens_h,
      inp.scale, k_scale=ks, v_scale=vs, seq_lens=dev["sl"] if seq_lens is None else seq_lens, out=out,
      lse_out=lse, **kw)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()


def expect(status, fn):
    import paged_kv_gqa_amd as pkv
    with pytest.raises(pkv.PkvError) as e:
        fn()
    log("  rejected: %s" % e.value)
    assert e.value.status == status and "PKV_VALIDATE" in str(e.value)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_valid_steps_give_the_same_bits(fmt, monkeypatch):
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16, q_len=2)
    inp = synth.make_inputs(c, seed=3, slack_pages=2, seq_lens=[max(2, L) for L in SEQ])
    dev = device_inputs(inp)
    T = 64 if fmt == "fp8" else 48
    a = decode(inp, dev, runner(inp, T=T))
    monkeypatch.setenv("PKV_VALIDATE", "1")
    b = decode(inp, dev, runner(inp, T=T))
    d = decode(inp, dev, runner(inp, device_plan=True))
    monkeypatch.setenv("PKV_VALIDATE", "0")
    e = decode(inp, dev, runner(inp, device_plan=True))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(d[0], e[0]) and np.array_equal(d[1], e[1])
    assert not np.isnan(a[1]).any()


def test_page_outside_the_cache_is_rejected(monkeypatch):
    inp = synth.make_inputs(cfg(), seed=4, slack_pages=2, seq_lens=SEQ)
    last = inp.k_cache.shape[0] - 1
    inp.block_table[5, 3] = last          # a real page, but past the num_pages passed below
    dev = device_inputs(inp)
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-1, lambda: decode(inp, dev, pages=last))


def test_short_sequence_is_rejected(monkeypatch):
    """Device lengths below max(1, q_len); the host plan was made from valid ones."""
    import torch
    inp = synth.make_inputs(cfg(q_len=2), seed=5, slack_pages=1, seq_lens=[max(2, L) for L in SEQ])
    dev = device_inputs(inp)
    sl = dev["sl"].clone()
    sl[3] = 1
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-6, lambda: decode(inp, dev, seq_lens=sl))
    del torch


def test_plan_of_other_lengths_is_rejected(monkeypatch):
    """Device length of request 1 one tile longer than the host plan's: the block-table
    row holds real pages past its length, and the plan's tile count no longer fits."""
    inp = synth.make_inputs(cfg(), seed=6, slack_pages=1, seq_lens=SEQ)
    inp.block_table[1, 1:6] = inp.block_table[1, 0]
    dev = device_inputs(inp)
    sl = dev["sl"].clone()
    sl[1] = SEQ[1] + 64
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-1, lambda: decode(inp, dev, seq_lens=sl))


def test_length_past_the_block_table_is_rejected(monkeypatch):
    """Request 0's device length one token past its block-table row; the row holds real
    pages throughout and the next row's first entry is a real page too."""
    inp = synth.make_inputs(cfg(), seed=7, slack_pages=1, seq_lens=SEQ)
    inp.block_table[0, :] = inp.block_table[0, 0]
    dev = device_inputs(inp)
    sl = dev["sl"].clone()
    sl[0] = inp.block_table.shape[1] * inp.page_size + 1
    monkeypatch.setenv("PKV_VALIDATE", "1")
    r = runner(inp, device_plan=True)     # a device plan would follow the device lengths
    expect(-1, lambda: decode(inp, dev, r=r, seq_lens=sl))


def test_combine_reading_past_num_partials_is_rejected(monkeypatch):
    import torch
    import paged_kv_gqa_amd as pkv
    monkeypatch.setenv("PKV_VALIDATE", "1")
    rtb = torch.tensor([0, 2, 5], dtype=torch.int32, device="cuda")   # 5 tiles x 2 kv heads
    ws = torch.zeros(pkv.pkv_workspace_bytes(10, 4, 128), dtype=torch.uint8, device="cuda")
    out = torch.full((2, 1, 8, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    expect(-1, lambda: pkv.pkv_combine(workspace=ws, workspace_bytes=ws.numel(), num_partials=9,
                                       req_tile_base=rtb, batch=2, q_len=1, num_q_heads=8,
                                       num_kv_heads=2, head_dim=128, out=out))
    assert torch.isnan(out.float()).all()


def test_block_sparse_page_outside_the_cache_is_rejected(monkeypatch):
    import torch
    inp = synth.make_inputs(cfg(), seed=8, slack_pages=2, seq_lens=SEQ)
    last = inp.k_cache.shape[0] - 1
    inp.block_table[6, 2] = last
    dev = device_inputs(inp)
    mask = np.ones((inp.batch, inp.num_kv_heads, inp.block_table.shape[1]), np.uint8)
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-1, lambda: decode(inp, dev, pages=last, block_mask=torch.from_numpy(mask).cuda(),
                              block_mask_h=mask))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_kv_append_page_outside_the_cache_is_rejected(fmt, monkeypatch):
    import torch
    c = cfg(kv_format=fmt, page_size=64 if fmt == "fp8" else 16)
    inp = synth.make_inputs(c, seed=9, slack_pages=2, seq_lens=SEQ)
    last = inp.k_cache.shape[0] - 1
    b = 6
    inp.block_table[b, (SEQ[b] - 1) // inp.page_size] = last     # the page of its new token
    dev = device_inputs(inp)
    kn_h, vn_h, _ = synth.new_token_rows(inp, seed=2)
    as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    r = runner(inp)
    # views of the whole cache: the "bad" page is real memory past num_pages = last
    k, v = dev["k"][:last], dev["v"][:last]
    before = k.view(torch.int16).cpu().numpy().copy() if fmt == "bf16" else k.cpu().numpy().copy()
    ks = None if dev["ks"] is None else dev["ks"][:last]
    vs = None if dev["vs"] is None else dev["vs"][:last]
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-1, lambda: r.append(as_bf16(kn_h), as_bf16(vn_h), k, v, dev["bt"], dev["sl"],
                                k_scale=ks, v_scale=vs))
    after = k.view(torch.int16).cpu().numpy() if fmt == "bf16" else k.cpu().numpy()
    assert np.array_equal(before, after)


def test_prefill_page_outside_the_cache_is_rejected(monkeypatch):
    import torch
    import paged_kv_gqa_amd as pkv
    p = synth.make_prefill_inputs(dict(name="prefill", batch=0, q_lens=("const", 1),
                                       prefix=("const", 0), num_q_heads=8, num_kv_heads=2,
                                       head_dim=128, page_size=16, kv_format="bf16"),
                                  seed=10, q_lens=[40, 70], prefix=[5, 30], slack_pages=2)
    c = p.cache
    last = c.k_cache.shape[0] - 1
    c.block_table[1, 4] = last
    dev = device_inputs(c)
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(p.cu_q).cuda()
    kl = torch.from_numpy(c.seq_lens).cuda()
    out = torch.full_like(q, float("nan"))
    r = pkv.PagedPrefill(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, kv_format="bf16")
    monkeypatch.setenv("PKV_VALIDATE", "1")
    expect(-1, lambda: r(q, cu, kl, dev["bt"], p.q_lens, c.seq_lens, c.scale, k_cache=dev["k"][:last],
                         v_cache=dev["v"][:last], out=out))
    assert torch.isnan(out.float()).all()
