"""Argument checks of the runners (PagedDecode, PagedDecode.append, PagedPrefill).

The runners hand raw device addresses to kernels that assume a dtype, a shape and a
contiguous layout, so a wrong tensor must be refused in Python before anything is
enqueued: an int64 block table, a transposed q, a cache of another width, scales of
another dtype. Each case below raises before the library is called (needs a GPU only
to build CUDA tensors).
"""

import numpy as np
import pytest

import synth
from tests.gpu_util import device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd as pkv
    c = dict(name="args", batch=0, seq_lens=(1,), q_len=2, num_q_heads=8, num_kv_heads=2,
             head_dim=128, page_size=64, kv_format="fp8")
    inp = synth.make_inputs(c, seed=1, slack_pages=1, seq_lens=[2, 70, 300])
    dev = device_inputs(inp)
    r = pkv.PagedDecode(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, kv_format="fp8",
                        q_len=2, tile_tokens=64, num_workers=3)
    return torch, pkv, inp, dev, r


def call(setup, **over):
    torch, pkv, inp, dev, r = setup
    a = dict(q=dev["q"], k=dev["k"], v=dev["v"], bt=dev["bt"], seq_lens_h=inp.seq_lens,
             k_scale=dev["ks"], v_scale=dev["vs"], seq_lens=dev["sl"], out=None, lse_out=None)
    a.update(over)
    return r(a["q"], a["k"], a["v"], a["bt"], a["seq_lens_h"], inp.scale, k_scale=a["k_scale"],
             v_scale=a["v_scale"], seq_lens=a["seq_lens"], out=a["out"], lse_out=a["lse_out"])


def test_valid_arguments_run(setup):
    torch = setup[0]
    out = call(setup)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (3, 2, 8, 128) and torch.isfinite(out.float()).all()


@pytest.mark.parametrize("case,exc,match", [
    ("bt_int64", TypeError, "block_table has dtype"),
    ("q_transposed", ValueError, "q must be contiguous"),
    ("q_float32", TypeError, "q has dtype"),
    ("q_wrong_heads", ValueError, "q has shape"),
    ("k_wrong_page", ValueError, "k_cache has shape"),
    ("v_fewer_pages", ValueError, "v_cache has shape"),
    ("scale_float16", TypeError, "k_scale has dtype"),
    ("scale_missing", TypeError, "v_scale must be a CUDA tensor"),
    ("seq_lens_int64", TypeError, "seq_lens has dtype"),
    ("seq_lens_h_short", ValueError, "seq_lens_h has 2 entries"),
    ("out_float32", TypeError, "out has dtype"),
    ("lse_wrong_shape", ValueError, "lse_out has shape"),
    ("bt_on_host", TypeError, "block_table must be a CUDA tensor"),
])
def test_decode_rejects(setup, case, exc, match):
    torch, pkv, inp, dev, r = setup
    q = dev["q"]
    over = {
        "bt_int64": dict(bt=dev["bt"].long()),
        "q_transposed": dict(q=q.transpose(1, 2).contiguous().transpose(1, 2)),
        "q_float32": dict(q=q.float()),
        "q_wrong_heads": dict(q=q[:, :, :4].contiguous()),
        "k_wrong_page": dict(k=dev["k"].reshape(dev["k"].shape[0], 2, 32, 256)),
        "v_fewer_pages": dict(v=dev["v"][:-1]),
        "scale_float16": dict(k_scale=dev["ks"].half()),
        "scale_missing": dict(v_scale=None),
        "seq_lens_int64": dict(seq_lens=dev["sl"].long()),
        "seq_lens_h_short": dict(seq_lens_h=inp.seq_lens[:2]),
        "out_float32": dict(out=torch.empty(q.shape, device=q.device)),
        "lse_wrong_shape": dict(lse_out=torch.empty((3, 2, 4), device=q.device)),
        "bt_on_host": dict(bt=dev["bt"].cpu()),
    }[case]
    with pytest.raises(exc, match=match):
        call(setup, **over)


def test_append_rejects(setup):
    torch, pkv, inp, dev, r = setup
    kn_h, vn_h, qn_h = synth.new_token_rows(inp, seed=3)
    as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    kn, vn = as_bf16(kn_h), as_bf16(vn_h)
    k, v = dev["k"].clone(), dev["v"].clone()
    before = k.cpu().numpy().copy()
    with pytest.raises(ValueError, match="k_new has shape"):
        r.append(kn[:, :1].contiguous(), vn, k, v, dev["bt"], dev["sl"], k_scale=dev["ks"],
                 v_scale=dev["vs"])
    with pytest.raises(TypeError, match="v_new has dtype"):
        r.append(kn, vn.float(), k, v, dev["bt"], dev["sl"], k_scale=dev["ks"], v_scale=dev["vs"])
    with pytest.raises(ValueError, match="come in pairs"):
        r.append(kn, vn, k, v, dev["bt"], dev["sl"], q=as_bf16(qn_h), k_scale=dev["ks"],
                 v_scale=dev["vs"])
    cos = torch.zeros((500, 64), device="cuda")
    with pytest.raises(ValueError, match="rope_sin has shape"):
        r.append(kn, vn, k, v, dev["bt"], dev["sl"], rope_cos=cos, rope_sin=cos[:, :32].contiguous(),
                 k_scale=dev["ks"], v_scale=dev["vs"])
    torch.cuda.synchronize()
    assert np.array_equal(before, k.cpu().numpy())      # nothing was written


def test_prefill_rejects():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd as pkv
    p = synth.make_prefill_inputs(dict(name="prefill", batch=0, q_lens=("const", 1),
                                       prefix=("const", 0), num_q_heads=8, num_kv_heads=2,
                                       head_dim=128, page_size=16, kv_format="bf16"),
                                  seed=2, q_lens=[40, 7], prefix=[5, 30])
    c = p.cache
    dev = device_inputs(c)
    q = torch.from_numpy(p.q.view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(p.cu_q).cuda()
    kl = torch.from_numpy(c.seq_lens).cuda()
    r = pkv.PagedPrefill(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16)
    run = lambda **o: r(o.get("q", q), o.get("cu", cu), o.get("kl", kl), o.get("bt", dev["bt"]),
                        p.q_lens, c.seq_lens, c.scale, k_cache=o.get("k", dev["k"]),
                        v_cache=dev["v"], out=o.get("out"), lse=o.get("lse"))
    out = run()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    with pytest.raises(TypeError, match="cu_q has dtype"):
        run(cu=cu.long())
    with pytest.raises(ValueError, match="q has shape"):
        run(q=q.reshape(q.shape[0], 4, 256))
    with pytest.raises(ValueError, match="kv_lens has shape"):
        run(kl=kl[:1])
    with pytest.raises(TypeError, match="k_cache has dtype"):
        run(k=dev["k"].float())
    with pytest.raises(ValueError, match="lse has shape"):
        run(lse=torch.empty((q.shape[0], 4), device="cuda"))
