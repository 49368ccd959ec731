"""pkv_decode_noalloc (the decode step for callers that cannot allocate) against the
existing entry points pkv_decode_partial + pkv_combine, through the C ABI on an
MI355X: two calls in a row on the library's shared device array, the second with a
smaller batch (and a smaller partial count) than the first, each bit-identical to the
workspace path and within the contract's tolerance of the fp64 oracle."""

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import device_inputs, log, max_abs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_gqa_amd  # noqa: F401  (fails loudly without the built library)


def step_args(inp, dev, T=0, W=0):
    """Host plan for the batch, copied to the device; the keyword arguments of
    pkv_decode_partial / pkv_decode_noalloc without the workspace."""
    import torch
    import paged_kv_gqa_amd as pkv
    W = W or pkv.pkv_default_num_workers(0, inp.kv_format, inp.head_dim)
    T, N, NP = pkv.pkv_plan_query(inp.seq_lens, inp.q_len, inp.num_q_heads, inp.num_kv_heads,
                                  inp.head_dim, inp.page_size, inp.kv_format, T, W)
    items, offs, rtb = pkv.pkv_plan(inp.seq_lens, inp.q_len, inp.num_kv_heads, T, W, num_items=N)
    plan = [torch.from_numpy(x).cuda() for x in (items, offs, rtb)]
    kw = dict(q=dev["q"], k_cache=dev["k"], v_cache=dev["v"], k_scale=dev["ks"], v_scale=dev["vs"],
              block_table=dev["bt"], seq_lens=dev["sl"], items=plan[0], worker_offsets=plan[1],
              req_tile_base=plan[2], num_items=N, num_partials=NP, num_pages=int(dev["k"].shape[0]),
              batch=inp.batch, q_len=inp.q_len, num_q_heads=inp.num_q_heads,
              num_kv_heads=inp.num_kv_heads, head_dim=inp.head_dim, page_size=inp.page_size,
              bt_stride=int(inp.block_table.shape[1]), kv_format=inp.kv_format, tile_tokens=T,
              num_workers=W, scale=inp.scale)
    return kw, plan


def run_both(inp, T=0, W=0):
    """(out bits, lse) of the workspace path and of pkv_decode_noalloc, same inputs."""
    import torch
    import paged_kv_gqa_amd as pkv
    dev = device_inputs(inp)
    kw, _plan = step_args(inp, dev, T, W)
    M = (inp.num_q_heads // inp.num_kv_heads) * inp.q_len
    nbytes = pkv.pkv_workspace_bytes(max(kw["num_partials"], 1), M, inp.head_dim)
    assert nbytes <= pkv.PKV_NOALLOC_SCRATCH_BYTES
    shape = (inp.batch, inp.q_len, inp.num_q_heads)
    outs = []
    for noalloc in (False, True):
        out = torch.empty(shape + (inp.head_dim,), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(shape, dtype=torch.float32, device="cuda")
        if noalloc:
            pkv.pkv_decode_noalloc(out=out, lse_out=lse, **kw)
        else:
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            pkv.pkv_decode_partial(workspace=ws, workspace_bytes=nbytes, **kw)
            pkv.pkv_combine(workspace=ws, workspace_bytes=nbytes, num_partials=kw["num_partials"],
                            req_tile_base=kw["req_tile_base"], batch=inp.batch, q_len=inp.q_len,
                            num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                            head_dim=inp.head_dim, out=out, lse_out=lse)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy().view(np.uint16), out.float().cpu().numpy(),
                     lse.cpu().numpy()))
    return outs


def check_call(inp, tol, T=0, W=0, tag=""):
    (bits_ws, out_ws, lse_ws), (bits_na, out_na, lse_na) = run_both(inp, T, W)
    assert np.array_equal(bits_ws, bits_na), tag
    assert np.array_equal(lse_ws, lse_na), tag
    ref, ref_lse = oracle.decode_attention(inp)
    err, lerr = max_abs(out_na, ref), max_abs(lse_na, ref_lse)
    log("  %s: noalloc = workspace path bit for bit; vs oracle max_abs %.3e, lse %.3e" % (tag, err, lerr))
    assert np.isfinite(out_na).all() and err <= tol and lerr <= 1e-3, tag


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_noalloc_matches_workspace_path_on_two_calls(fmt):
    P = 64 if fmt == "fp8" else 16
    tol = 3e-2 if fmt == "fp8" else 1e-2
    big = dict(name="na_big", batch=0, seq_lens=(1,), q_len=2, num_q_heads=32, num_kv_heads=8,
               head_dim=128, page_size=P, kv_format=fmt)
    inp1 = synth.make_inputs(big, seed=11, poison=True, slack_pages=2,
                             seq_lens=[2, 70, 700, 3000, 5000, 9000])
    log("no-alloc %s: first call, B=%d" % (fmt, inp1.batch))
    check_call(inp1, tol, T=256, tag="%s first (B=6, T=256)" % fmt)
    small = dict(big, name="na_small", num_q_heads=16, num_kv_heads=2, q_len=4)
    inp2 = synth.make_inputs(small, seed=12, poison=True, slack_pages=1, seq_lens=[4, 100, 1500])
    log("no-alloc %s: second call, smaller (B=%d)" % (fmt, inp2.batch))
    check_call(inp2, tol, tag="%s second (B=3, M=32, automatic tile)" % fmt)
