"""The C-ABI library on the host (no GPU calls): symbols, version, the native planner
bit for bit against the reference planner, and the argument checks that return
before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_gqa_amd as pkv
import synth
from oracle import plan as ref_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        text = f.read()
    # declarations: a return type at the start of a line, then the function name
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(pkv_[a-z_]+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) == 19
    lib = ctypes.CDLL(pkv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
        assert hasattr(pkv, n), n          # and the binding mirrors it


def test_version_and_status_strings():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        ver = int(re.search(r"#define PKV_ABI_VERSION (\d+)", f.read()).group(1))
    assert pkv.pkv_abi_version() == ver
    for code in range(0, -7, -1):
        assert pkv.pkv_status_string(code) not in ("", "unknown status")
    assert pkv.pkv_status_string(-99) == "unknown status"


def native_plan(sl, q_len, Hq, Hkv, D, P, fmt, T, W):
    T, N, NP = pkv.pkv_plan_query(sl, q_len, Hq, Hkv, D, P, fmt, T, W)
    assert NP == N
    items, offs, rtb = pkv.pkv_plan(sl, q_len, Hkv, T, W, num_items=N)
    return T, items, offs, rtb


def assert_same_plan(sl, q_len, Hq, Hkv, D, P, fmt, T, W):
    Tn, items, offs, rtb = native_plan(sl, q_len, Hq, Hkv, D, P, fmt, T, W)
    ref = ref_plan.plan(sl, q_len, Hq, Hkv, D, P, fmt, T, W)
    assert Tn == ref["tile_tokens"]
    assert np.array_equal(items, ref["items"])
    assert np.array_equal(offs, ref["worker_offsets"])
    assert np.array_equal(rtb, ref["req_tile_base"])


@pytest.mark.parametrize("name", list(synth.ALL))
@pytest.mark.parametrize("W", [256, 512, 1024])
def test_plan_matches_reference_on_workloads(name, W):
    cfg = synth.ALL[name]
    sl = synth.draw_seq_lens(cfg, np.random.default_rng(0))
    args = (sl, cfg["q_len"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"],
            cfg["page_size"], cfg["kv_format"])
    assert_same_plan(*args, 0, W)
    quantum = ref_plan.tile_quantum(cfg["page_size"], cfg["kv_format"])
    assert_same_plan(*args, quantum * 8, W)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.integers(1, 5000), min_size=1, max_size=12), st.integers(1, 4),
       st.sampled_from([16, 32, 64]), st.integers(1, 40), st.integers(0, 6), st.sampled_from(["bf16", "fp8"]),
       st.integers(1, 4))
def test_plan_matches_reference_fuzz(sl, Hkv, P, W, k, fmt, q_len):
    sl = [max(L, q_len) for L in sl]
    T = 0 if k == 0 else ref_plan.tile_quantum(P, fmt) * k
    assert_same_plan(sl, q_len, Hkv * min(4, 16 // q_len), Hkv, 128, P, fmt, T, W)


def test_plan_of_empty_batch():
    T, N, NP = pkv.pkv_plan_query([], 1, 4, 1, 64, 16, "bf16", 0, 8)
    assert N == 0 and NP == 0
    items, offs, rtb = pkv.pkv_plan([], 1, 1, T, 8, num_items=0)
    assert offs.tolist() == [0] * 9 and rtb.tolist() == [0]


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), pkv.PKV_ERR_UNSUPPORTED),
    (dict(page_size=24), pkv.PKV_ERR_UNSUPPORTED),
    (dict(num_q_heads=6, num_kv_heads=4), pkv.PKV_ERR_UNSUPPORTED),
    (dict(q_len=5), pkv.PKV_ERR_UNSUPPORTED),
    (dict(num_q_heads=32, num_kv_heads=1, q_len=4), pkv.PKV_ERR_UNSUPPORTED),  # M = 128 > 64
    (dict(tile_tokens=24), pkv.PKV_ERR_UNSUPPORTED),
    (dict(num_workers=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(tile_tokens=-16), pkv.PKV_ERR_INVALID_ARG),
    (dict(kv_format=7), pkv.PKV_ERR_INVALID_ARG),
    (dict(seq_lens=[5, 0]), pkv.PKV_ERR_SEQ),
    (dict(seq_lens=[5, 2], q_len=3), pkv.PKV_ERR_SEQ),
])
def test_plan_query_errors(kw, status):
    a = dict(seq_lens=[17, 64], q_len=1, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
             kv_format="bf16", tile_tokens=0, num_workers=4)
    a.update(kw)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_query(a["seq_lens"], a["q_len"], a["num_q_heads"], a["num_kv_heads"], a["head_dim"],
                           a["page_size"], a["kv_format"], a["tile_tokens"], a["num_workers"])
    assert e.value.status == status
    assert pkv.pkv_last_error() != ""


def test_plan_errors():
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([3, 0], 1, 1, 16, 2, num_items=1)
    assert e.value.status == pkv.PKV_ERR_SEQ
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([3], 1, 1, 0, 2, num_items=1)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan([3], 1, 1, 16, 0, num_items=1)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG


def test_workspace_bytes():
    o = 10 * 4 * 128 * 4
    l = 10 * 4 * 4
    assert pkv.pkv_workspace_bytes(10, 4, 128) == (o + 255) // 256 * 256 + (l + 255) // 256 * 256
    assert pkv.pkv_workspace_bytes(0, 4, 128) == 0
    with pytest.raises(pkv.PkvError):
        pkv.pkv_workspace_bytes(-1, 4, 128)


# Fake device addresses: every check below fails before the library makes a HIP call.
A = 1 << 20


def decode_kwargs(**kw):
    base = dict(q=A, k_cache=2 * A, v_cache=3 * A, block_table=4 * A, seq_lens=5 * A, items=6 * A,
                worker_offsets=7 * A, req_tile_base=8 * A, workspace=9 * A, workspace_bytes=1 << 30,
                num_items=4, num_partials=4, num_pages=8, batch=2, q_len=1, num_q_heads=8,
                num_kv_heads=2, head_dim=128, page_size=16, bt_stride=4, kv_format="bf16",
                tile_tokens=32, num_workers=2, scale=0.1, stream=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,status", [
    (dict(q=A + 8), pkv.PKV_ERR_ALIGNMENT),
    (dict(workspace=9 * A + 4), pkv.PKV_ERR_ALIGNMENT),
    (dict(items=6 * A + 4), pkv.PKV_ERR_ALIGNMENT),
    (dict(workspace_bytes=100), pkv.PKV_ERR_WORKSPACE),
    (dict(head_dim=80), pkv.PKV_ERR_UNSUPPORTED),
    (dict(tile_tokens=24), pkv.PKV_ERR_UNSUPPORTED),
    (dict(kv_format="fp8"), pkv.PKV_ERR_UNSUPPORTED),     # tile 32: the fp8 quantum is lcm(16, 64)
    (dict(kv_format="fp8", page_size=64, tile_tokens=64), pkv.PKV_ERR_INVALID_ARG),  # no scales
    (dict(k_scale=10 * A), pkv.PKV_ERR_INVALID_ARG),                                  # bf16 with scales
    (dict(q=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_workers=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_partials=2), pkv.PKV_ERR_INVALID_ARG),
    (dict(bt_stride=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), pkv.PKV_ERR_INVALID_ARG),
])
def test_decode_partial_argument_errors(kw, status):
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_partial(**decode_kwargs(**kw))
    assert e.value.status == status


def test_decode_partial_struct_size_checked():
    a = pkv.DecodeArgs()
    a.struct_size = 8
    assert pkv._lib.pkv_decode_partial(ctypes.byref(a), None) == pkv.PKV_ERR_INVALID_ARG
    assert pkv._lib.pkv_decode_partial(None, None) == pkv.PKV_ERR_INVALID_ARG


def test_decode_partial_without_items_is_a_no_op():
    pkv.pkv_decode_partial(**decode_kwargs(num_items=0, num_partials=0))


@pytest.mark.parametrize("name", ["q", "k_cache", "k_scale", "block_table", "seq_lens", "items",
                                  "workspace"])
def test_host_arrays_are_not_device_arguments(name):
    """A numpy array or CPU tensor holds pageable host memory the kernels cannot read;
    the binding refuses it before anything reaches the library."""
    import torch
    for host in (np.zeros(64, np.float32), torch.zeros(64)):
        with pytest.raises(TypeError, match=name):
            pkv.pkv_decode_partial(**decode_kwargs(**{name: host}))
    with pytest.raises(TypeError, match="out"):
        pkv.pkv_combine(workspace=9 * A, workspace_bytes=1 << 30, num_partials=4, req_tile_base=8 * A,
                        batch=2, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                        out=np.zeros(8, np.uint16), stream=0)


def test_abi1_struct_size_is_accepted():
    """A caller built against ABI 1 passes the struct without tile_tokens_dev."""
    v1 = pkv.DecodeArgs.tile_tokens_dev.offset
    a = pkv.DecodeArgs()
    kw = decode_kwargs(num_items=0, num_partials=0)
    for name in ("batch", "q_len", "num_q_heads", "num_kv_heads", "head_dim", "page_size",
                 "bt_stride", "tile_tokens", "num_workers", "scale"):
        setattr(a, name, kw[name])
    a.tile_tokens_dev = 8 * A            # beyond an ABI 1 struct: must not be read
    a.struct_size = v1
    assert pkv._lib.pkv_decode_partial(ctypes.byref(a), None) == pkv.PKV_OK
    a.struct_size = v1 - 8
    assert pkv._lib.pkv_decode_partial(ctypes.byref(a), None) == pkv.PKV_ERR_INVALID_ARG


def test_device_tile_replaces_the_host_tile_check():
    # tile_tokens 24 is no multiple of 16, but with tile_tokens_dev it is not used
    pkv.pkv_decode_partial(**decode_kwargs(num_items=0, num_partials=0, tile_tokens=24,
                                           tile_tokens_dev=10 * A))
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_partial(**decode_kwargs(tile_tokens_dev=10 * A + 2))
    assert e.value.status == pkv.PKV_ERR_ALIGNMENT


def test_plan_device_scratch_bytes():
    # fixed tile: the candidate block plus one placement per remainder item
    assert pkv.pkv_plan_device_scratch_bytes(0, 8, 16, "bf16", 64, 512, 100) == 256
    assert pkv.pkv_plan_device_scratch_bytes(128, 8, 16, "bf16", 64, 512, 100) == 256 + 8 * 128 * 8
    # automatic tile: 13 candidates (16 .. 65536), each with placements and a whole plan
    r = lambda x: (x + 255) // 256 * 256
    B, H, W, cap = 128, 8, 512, 1000
    plan = r(16 * cap) + r(4 * (W + 1)) + r(4 * (B + 1)) + 256
    assert pkv.pkv_plan_device_scratch_bytes(B, H, 16, "bf16", 0, W, cap) == \
        r(256 + 13 * 8 * B * H) + 13 * plan
    # fp8 (quantum 64): 11 candidates
    assert pkv.pkv_plan_device_scratch_bytes(B, H, 64, "fp8", 0, W, cap) == \
        r(256 + 11 * 8 * B * H) + 11 * plan
    with pytest.raises(pkv.PkvError):
        pkv.pkv_plan_device_scratch_bytes(-1, 8, 16, "bf16", 0, 512, 10)


def plan_device_kwargs(**kw):
    base = dict(seq_lens=A, batch=4, q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
                page_size=16, kv_format="bf16", tile_tokens=0, num_workers=512, max_items=100,
                items=2 * A, worker_offsets=3 * A, req_tile_base=4 * A, info=5 * A, scratch=6 * A,
                scratch_bytes=1 << 20, stream=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,status", [
    (dict(num_workers=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_workers=1025), pkv.PKV_ERR_UNSUPPORTED),
    (dict(batch=4097), pkv.PKV_ERR_UNSUPPORTED),
    (dict(batch=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(max_items=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(max_items=1 << 30), pkv.PKV_ERR_UNSUPPORTED),
    (dict(tile_tokens=24), pkv.PKV_ERR_UNSUPPORTED),
    (dict(tile_tokens=-16), pkv.PKV_ERR_INVALID_ARG),
    (dict(tile_tokens=(1 << 18) + 16), pkv.PKV_ERR_UNSUPPORTED),
    (dict(head_dim=96), pkv.PKV_ERR_UNSUPPORTED),
    (dict(info=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(seq_lens=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(items=2 * A + 4), pkv.PKV_ERR_ALIGNMENT),
    (dict(scratch=6 * A + 8), pkv.PKV_ERR_ALIGNMENT),
    (dict(tile_tokens=64, scratch_bytes=256 + 8 * 4 * 2 - 1), pkv.PKV_ERR_WORKSPACE),
    (dict(scratch_bytes=1000), pkv.PKV_ERR_WORKSPACE),
])
def test_plan_device_argument_errors(kw, status):
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_plan_device(**plan_device_kwargs(**kw))
    assert e.value.status == status


@pytest.mark.parametrize("fmt,P,q_len", [("bf16", 16, 1), ("bf16", 32, 4), ("fp8", 64, 2)])
def test_block_sparse_lengths_match_the_attended_pages(fmt, P, q_len):
    c = dict(name="s", batch=6, seq_lens=(4, 15, 16, 17, 100, 700), q_len=q_len, num_q_heads=8,
             num_kv_heads=2, head_dim=64, page_size=P, kv_format=fmt)
    inp = synth.make_inputs(c, seed=1)
    for keep in (0.0, 0.3, 1.0):
        mask = synth.make_block_mask(inp, keep, seed=2)
        got = pkv.pkv_block_sparse_lengths(inp.seq_lens, mask, 2, q_len, P)
        att = synth.attended_pages(inp, mask)
        want = [sum(min(P, int(inp.seq_lens[b]) - p * P) for p in att[b][g])
                for b in range(inp.batch) for g in range(2)]
        assert got.tolist() == want


def test_block_sparse_lengths_errors():
    m = np.ones((2, 1, 4), np.uint8)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_block_sparse_lengths([5, 0], m, 1, 1, 16)
    assert e.value.status == pkv.PKV_ERR_SEQ
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_block_sparse_lengths([5, 65], m, 1, 1, 16)      # 5 pages, mask rows of 4
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(batch=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(mask_stride=3), pkv.PKV_ERR_INVALID_ARG),              # shorter than bt_stride
    (dict(num_pages=1 << 29), pkv.PKV_ERR_UNSUPPORTED),           # x 8 kv heads > int32
    (dict(block_mask=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(bt_out=7 * A + 2), pkv.PKV_ERR_ALIGNMENT),
])
def test_block_sparse_compact_errors(kw, status):
    base = dict(block_table=A, seq_lens=2 * A, block_mask=3 * A, batch=2, num_kv_heads=8, q_len=1,
                page_size=16, bt_stride=4, mask_stride=4, num_pages=64, bt_out=7 * A,
                seq_lens_out=8 * A, stream=0)
    base.update(kw)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_block_sparse_compact(**base)
    assert e.value.status == status


def test_request_split_must_divide_the_batch():
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_decode_partial(**decode_kwargs(request_split=3))
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_combine_split(workspace=9 * A, workspace_bytes=1 << 30, num_partials=4,
                              req_tile_base=8 * A, batch=6, q_len=1, num_q_heads=4, num_kv_heads=1,
                              head_dim=128, request_split=4, out=A, stream=0)
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG


def test_prefill_plan_lists_tiles_heaviest_first():
    q_lens, kv_lens = [70, 1, 130], [70, 40, 200]
    items = pkv.pkv_prefill_plan(q_lens, kv_lens, 16, 2)       # G = 8: 2 head groups of 4
    want = []
    for b, (n, L) in enumerate(zip(q_lens, kv_lens)):
        for t0 in range(0, n, 64):
            keys = L - n + min(t0 + 64, n)
            for g in range(2):
                for hg in range(2):
                    want.append((-keys, b, g, hg, t0))
    want.sort()
    assert items.tolist() == [[b, g, hg, t0] for _, b, g, hg, t0 in want]
    assert pkv.pkv_prefill_plan_size(q_lens, 16, 2) == len(want)
    assert pkv.pkv_prefill_plan([3], [3], 4, 4).tolist() == [[0, 0, 0, 0], [0, 1, 0, 0], [0, 2, 0, 0],
                                                             [0, 3, 0, 0]]


def test_prefill_plan_errors():
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefill_plan([5], [4], 8, 2)                    # kv shorter than the queries
    assert e.value.status == pkv.PKV_ERR_INVALID_ARG
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefill_plan([5], [5], 6, 2)                    # G = 3
    assert e.value.status == pkv.PKV_ERR_UNSUPPORTED


def prefill_kwargs(**kw):
    base = dict(q=A, cu_q=2 * A, kv_lens=3 * A, block_table=4 * A, items=5 * A, num_items=4,
                k_cache=6 * A, v_cache=7 * A, out=8 * A, num_pages=16, batch=2, num_q_heads=8,
                num_kv_heads=2, head_dim=128, page_size=16, bt_stride=4, kv_format="bf16",
                scale=0.1, stream=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(head_dim=96), pkv.PKV_ERR_UNSUPPORTED),
    (dict(page_size=8), pkv.PKV_ERR_UNSUPPORTED),
    (dict(kv_format="fp8"), pkv.PKV_ERR_INVALID_ARG),                  # no scales (page 16)
    (dict(kv_format="fp8", page_size=64), pkv.PKV_ERR_INVALID_ARG),    # no scales
    (dict(num_q_heads=6), pkv.PKV_ERR_UNSUPPORTED),                    # G = 3
    (dict(items=5 * A + 4), pkv.PKV_ERR_ALIGNMENT),
    (dict(scale=float("inf")), pkv.PKV_ERR_INVALID_ARG),
])
def test_prefill_argument_errors(kw, status):
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_prefill(**prefill_kwargs(**kw))
    assert e.value.status == status


def test_prefill_without_items_is_a_no_op():
    pkv.pkv_prefill(**prefill_kwargs(num_items=0))


def append_kwargs(**kw):
    base = dict(k_new=A, v_new=2 * A, k_cache=3 * A, v_cache=4 * A, block_table=5 * A,
                seq_lens=6 * A, num_pages=8, batch=2, q_len=1, num_q_heads=8, num_kv_heads=2,
                head_dim=128, page_size=16, bt_stride=4, kv_format="bf16", stream=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,status", [
    (dict(k_new=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(kv_format="fp8", page_size=64), pkv.PKV_ERR_INVALID_ARG),              # no scales
    (dict(k_scale=7 * A), pkv.PKV_ERR_INVALID_ARG),                               # bf16 with scales
    (dict(rope_cos=7 * A), pkv.PKV_ERR_INVALID_ARG),                              # one table only
    (dict(q=7 * A), pkv.PKV_ERR_INVALID_ARG),                                     # q without q_out
    (dict(rope_cos=7 * A, rope_sin=8 * A, max_pos=63), pkv.PKV_ERR_INVALID_ARG),  # < 4 x 16
    (dict(k_new=A + 4), pkv.PKV_ERR_ALIGNMENT),
    (dict(head_dim=96), pkv.PKV_ERR_UNSUPPORTED),
    (dict(q_len=5), pkv.PKV_ERR_UNSUPPORTED),
    (dict(bt_stride=0), pkv.PKV_ERR_INVALID_ARG),
])
def test_kv_append_argument_errors(kw, status):
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_kv_append(**append_kwargs(**kw))
    assert e.value.status == status


def test_kv_append_empty_batch_is_a_no_op():
    pkv.pkv_kv_append(**append_kwargs(batch=0))


@pytest.mark.parametrize("kw,status", [
    (dict(out=A + 2), pkv.PKV_ERR_ALIGNMENT),
    (dict(workspace_bytes=16), pkv.PKV_ERR_WORKSPACE),
    (dict(head_dim=32), pkv.PKV_ERR_UNSUPPORTED),
    (dict(out=None), pkv.PKV_ERR_INVALID_ARG),
    (dict(num_partials=-1), pkv.PKV_ERR_INVALID_ARG),
])
def test_combine_argument_errors(kw, status):
    base = dict(workspace=9 * A, workspace_bytes=1 << 30, num_partials=4, req_tile_base=8 * A, batch=2,
                q_len=1, num_q_heads=8, num_kv_heads=2, head_dim=128, out=A, stream=0)
    base.update(kw)
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_combine(**base)
    assert e.value.status == status


def test_noalloc_rejects_partials_past_its_array():
    """pkv_decode_noalloc refuses, before any HIP call, a step whose partials would not
    fit the library's static device array."""
    import ctypes
    a = pkv.DecodeArgs()
    a.struct_size = ctypes.sizeof(pkv.DecodeArgs)
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = 1, 1, 32, 8, 128
    a.page_size, a.kv_format, a.tile_tokens, a.num_workers = 16, 0, 16, 1
    # 4 rows x (128 + 1) floats per partial: 2^15 partials need 64.5 MiB + alignment
    a.num_items = a.num_partials = 1 << 15
    st = pkv._lib.pkv_decode_noalloc(ctypes.byref(a), None, None, None)
    assert st == pkv.PKV_ERR_WORKSPACE
    assert "static scratch" in pkv.pkv_last_error()
