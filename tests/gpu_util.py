"""Helpers for the GPU tests: move a synth.DecodeInputs batch to the device and run
one decode step through the C ABI (via the ctypes binding)."""

import sys

import numpy as np


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(inp):
    import torch
    dev = torch.device("cuda", 0)
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if inp.kv_format == "bf16":
        k = torch.from_numpy(inp.k_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(inp.v_cache.view(np.int16)).view(torch.bfloat16).to(dev)
        ks = vs = None
    else:
        k = torch.from_numpy(inp.k_cache).to(dev)
        v = torch.from_numpy(inp.v_cache).to(dev)
        ks = torch.from_numpy(inp.k_scale).to(dev)
        vs = torch.from_numpy(inp.v_scale).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    return dict(q=q, k=k, v=v, ks=ks, vs=vs, bt=bt, sl=sl)


def make_runner(inp, tile_tokens=0, num_workers=0):
    import paged_kv_gqa_amd as pkv
    return pkv.PagedDecode(num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
                           head_dim=inp.head_dim, page_size=inp.page_size, kv_format=inp.kv_format,
                           q_len=inp.q_len, tile_tokens=tile_tokens, num_workers=num_workers)


def run_decode(inp, tile_tokens=0, num_workers=0, dev=None, runner=None):
    """Returns (out float32 numpy [B,Tq,Hq,D], lse float32 numpy [B,Tq,Hq], out bf16 bits)."""
    import torch
    dev = dev or device_inputs(inp)
    runner = runner or make_runner(inp, tile_tokens, num_workers)
    B = inp.batch
    lse = torch.empty((B, inp.q_len, inp.num_q_heads), dtype=torch.float32, device="cuda")
    out = runner(dev["q"], dev["k"], dev["v"], dev["bt"], inp.seq_lens, inp.scale,
                 k_scale=dev["ks"], v_scale=dev["vs"], seq_lens=dev["sl"], lse_out=lse)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return out.float().cpu().numpy(), lse.cpu().numpy(), bits


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def pages_past_two_gib(inp, dev):
    """Device copies with the cache's pages moved to physical indices whose byte offsets
    lie past 2^31: a cache of base + n pages whose first `base` pages are NaN (e4m3fn
    0x7F for fp8; scales NaN), pages base .. base+n-1 the original ones, and the block
    table shifted by base. Returns (moved dev dict, base, cache bytes per tensor)."""
    import torch
    fp8 = inp.kv_format != "bf16"
    page_bytes = inp.num_kv_heads * inp.page_size * inp.head_dim * (1 if fp8 else 2)
    base = (1 << 31) // page_bytes + 7
    n = dev["k"].shape[0]
    moved = dict(dev)
    for name in ("k", "v"):
        t = torch.empty((base + n,) + tuple(dev[name].shape[1:]), dtype=dev[name].dtype, device="cuda")
        if fp8:
            t.fill_(0x7F)
        else:
            t.fill_(float("nan"))
        t[base:] = dev[name]
        moved[name] = t
    if fp8:
        for name in ("ks", "vs"):
            t = torch.full((base + n,) + tuple(dev[name].shape[1:]), float("nan"), device="cuda")
            t[base:] = dev[name]
            moved[name] = t
    bt = inp.block_table.copy()
    bt[bt >= 0] += base
    moved["bt"] = torch.from_numpy(bt).cuda()
    return moved, base, moved["k"].numel() * moved["k"].element_size()
