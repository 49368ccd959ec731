"""Decode steps on side streams (needs an MI355X).

The runner enqueues everything on the current stream (or the one passed as
``stream=``), with one plan buffer per step from a ring that it recycles only after the
kernels that read it have completed. Here two runners work on two side streams at
once, each for more steps than the ring has buffers and with no host synchronisation
between steps, and every output must carry the same bits as one step on the default
stream: host plan, device plan and block-sparse steps.
"""

import numpy as np
import pytest

import synth
from tests.gpu_util import device_inputs, log

pytestmark = pytest.mark.gpu

STEPS = 7   # more than the runner's 3 plan buffers


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd as pkv
    c = dict(name="streams", batch=0, seq_lens=(1,), q_len=2, num_q_heads=16, num_kv_heads=2,
             head_dim=128, page_size=16, kv_format="bf16")
    inp = synth.make_inputs(c, seed=11, slack_pages=1,
                            seq_lens=[2, 17, 64, 100, 333, 1000, 2049, 5000])
    return torch, pkv, inp, device_inputs(inp)


def runner(pkv, inp, **kw):
    return pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                           head_dim=inp.head_dim, page_size=inp.page_size, kv_format=inp.kv_format,
                           q_len=inp.q_len, tile_tokens=kw.pop("T", 256), num_workers=kw.pop("W", 9),
                           **kw)


def bits(torch, out):
    return out.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("mode", ["host", "device", "sparse"])
def test_side_streams_match_the_default_stream(env, mode):
    torch, pkv, inp, dev = env
    mask = None
    if mode == "sparse":
        rng = np.random.default_rng(5)
        mask = (rng.random((inp.batch, inp.num_kv_heads, inp.block_table.shape[1])) < 0.5).astype(np.uint8)
    kw = dict(device_plan=(mode == "device"))

    def step(r, out, stream=None):
        extra = {} if mask is None else dict(block_mask=mask_d, block_mask_h=mask)
        r(dev["q"], dev["k"], dev["v"], dev["bt"], inp.seq_lens, inp.scale, seq_lens=dev["sl"],
          out=out, stream=stream, **extra)

    mask_d = None if mask is None else torch.from_numpy(mask).cuda()
    shape = (inp.batch, inp.q_len, inp.num_q_heads, inp.head_dim)
    ref = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    step(runner(pkv, inp, **kw), ref)
    torch.cuda.synchronize()
    ref_bits = bits(torch, ref)
    assert not np.isnan(ref.float().cpu().numpy()).any()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    r1, r2 = runner(pkv, inp, **kw), runner(pkv, inp, **kw)
    outs1 = [torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(STEPS)]
    outs2 = [torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(STEPS)]
    torch.cuda.synchronize()
    for i in range(STEPS):
        with torch.cuda.stream(s1):           # the stream as the current stream
            step(r1, outs1[i])
        step(r2, outs2[i], stream=s2)        # the stream as an argument
    torch.cuda.synchronize()
    for i in range(STEPS):
        assert np.array_equal(bits(torch, outs1[i]), ref_bits), (mode, "s1", i)
        assert np.array_equal(bits(torch, outs2[i]), ref_bits), (mode, "s2", i)
    log("  %s: %d steps on each of two side streams, bit-identical to the default stream"
        % (mode, STEPS))
