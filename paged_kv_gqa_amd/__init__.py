"""Python binding of libpkv.so: paged-KV GQA attention on MI355X.

Thin ctypes wrappers with the C ABI's names (argument marshalling only; every step
runs in the library): split-KV decode (host or device plan, partial kernel, combine),
block-sparse decode, the fused KV append, and variable-length prefill. On top of them:
- ``PagedDecode``, a per-step runner that plans on the host into mapped pinned memory
  the kernels read in place (or, with ``device_plan=True``, enqueues the device-side
  planner) and enqueues the kernels on the caller's stream;
- ``PagedPrefill``, which plans prefill tiles on the host and enqueues the prefill
  kernel.
PyTorch supplies device memory and streams.

The library is built in-tree (``python paged_kv_gqa_amd/_build.py``); importing this
package without it raises ImportError - there is no fallback path.
"""

import ctypes
import os

import numpy as np
# torch ships its own HIP runtime (soname libamdhip64.so.7). Loading it before the
# library makes libpkv.so bind to that same runtime, so the process holds one HIP/HSA
# runtime and torch's device pointers and streams are valid in the library.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

KV_BF16 = 0
KV_FP8_E4M3FN = 1
KV_FORMATS = {"bf16": KV_BF16, "fp8": KV_FP8_E4M3FN}

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_ALIGNMENT = -3
PKV_ERR_WORKSPACE = -4
PKV_ERR_HIP = -5
PKV_ERR_SEQ = -6

MAX_ROWS = 64  # largest (q heads per kv head) x (query tokens) per work item

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class PkvError(RuntimeError):
    def __init__(self, status, func, detail):
        super().__init__("%s failed: %s (%d): %s" % (func, _status_text(status), status, detail))
        self.status = status


class DecodeArgs(ctypes.Structure):
    """Mirror of ``pkv_decode_args`` (include/pkv.h)."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("items", ctypes.c_void_p), ("worker_offsets", ctypes.c_void_p),
        ("req_tile_base", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_items", ctypes.c_int64), ("num_partials", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("batch", ctypes.c_int), ("q_len", ctypes.c_int), ("num_q_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("page_size", ctypes.c_int),
        ("bt_stride", ctypes.c_int), ("kv_format", ctypes.c_int), ("tile_tokens", ctypes.c_int),
        ("num_workers", ctypes.c_int), ("scale", ctypes.c_float),
        ("tile_tokens_dev", ctypes.c_void_p), ("request_split", ctypes.c_int),
        ("out", ctypes.c_void_p), ("lse_out", ctypes.c_void_p),
    ]


class KvAppendArgs(ctypes.Structure):
    """Mirror of ``pkv_kv_append_args`` (include/pkv.h)."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("q", ctypes.c_void_p), ("q_out", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("num_pages", ctypes.c_int64),
        ("batch", ctypes.c_int), ("q_len", ctypes.c_int), ("num_q_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("page_size", ctypes.c_int),
        ("bt_stride", ctypes.c_int), ("kv_format", ctypes.c_int), ("max_pos", ctypes.c_int),
    ]


class PrefillArgs(ctypes.Structure):
    """Mirror of ``pkv_prefill_args`` (include/pkv.h)."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("cu_q", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("items", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("num_items", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("batch", ctypes.c_int), ("num_q_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
        ("head_dim", ctypes.c_int), ("page_size", ctypes.c_int), ("bt_stride", ctypes.c_int),
        ("kv_format", ctypes.c_int), ("scale", ctypes.c_float),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpkv.so is not built (expected at %s); run "
                          "`python paged_kv_gqa_amd/_build.py` from the repository root" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "pkv_abi_version": (ctypes.c_int, []),
        "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_plan_query": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, _i32p, _i64p, _i64p]),
        "pkv_plan": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
        "pkv_default_num_workers": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                   ctypes.POINTER(ctypes.c_int)]),
        "pkv_workspace_bytes": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_size_t)]),
        "pkv_decode_partial": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]),
        "pkv_plan_device_scratch_bytes": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                         ctypes.c_int64,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
        "pkv_plan_device": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
        "pkv_combine_split": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
        "pkv_block_sparse_compact": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
        "pkv_block_sparse_lengths": (ctypes.c_int, [ctypes.c_int, _i32p, ctypes.c_void_p, ctypes.c_int,
                                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p]),
        "pkv_kv_append": (ctypes.c_int, [ctypes.POINTER(KvAppendArgs), ctypes.c_void_p]),
        "pkv_prefill_plan_size": (ctypes.c_int, [ctypes.c_int, _i32p, ctypes.c_int, ctypes.c_int, _i64p]),
        "pkv_prefill_plan": (ctypes.c_int, [ctypes.c_int, _i32p, _i32p, ctypes.c_int, ctypes.c_int, _i32p]),
        "pkv_prefill": (ctypes.c_int, [ctypes.POINTER(PrefillArgs), ctypes.c_void_p]),
        "pkv_decode_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeArgs), ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]),
        "pkv_combine": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _status_text(status):
    return _lib.pkv_status_string(status).decode()


def _check(status, func):
    if status != PKV_OK:
        raise PkvError(status, func, _lib.pkv_last_error().decode())


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def _ptr(t, name="argument"):
    """Device address of a device-side argument: a CUDA tensor, an int address (device
    memory or mapped pinned host memory) or None. Anything else - a numpy array or a
    CPU tensor lives in pageable host memory the GPU cannot read - raises TypeError
    before the library sees it."""
    if t is None:
        return None
    if isinstance(t, (int, np.integer)) and not isinstance(t, bool):
        return int(t)
    if hasattr(t, "data_ptr") and getattr(t, "is_cuda", False):
        return t.data_ptr()
    raise TypeError("%s must be a CUDA tensor, a device-accessible address or None, not %s"
                    % (name, type(t).__name__ if not hasattr(t, "device") else "a tensor on %s" % t.device))


def _check_tensor(t, name, dtypes, shape, device):
    """Argument check of the runners, which pass raw device addresses to kernels that
    assume a layout: ``t`` must be a contiguous CUDA tensor on ``device``, of one of
    ``dtypes``, with ``shape`` (None = any extent). Raises TypeError or ValueError.
    The common case costs about a microsecond; the message is built only on failure."""
    try:
        if t.device == device and t.dtype in dtypes and t.is_contiguous():
            s = t.shape
            if len(s) == len(shape):
                for a, e in zip(s, shape):
                    if e is not None and a != e:
                        break
                else:
                    return
    except AttributeError:
        pass
    if not (hasattr(t, "data_ptr") and getattr(t, "is_cuda", False)):
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, the runner on %s" % (name, t.device, device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s; expected %s" % (name, t.dtype, " or ".join(map(str, dtypes))))
    if len(t.shape) != len(shape) or any(e is not None and int(a) != e for a, e in zip(t.shape, shape)):
        raise ValueError("%s has shape %s; expected [%s]" % (
            name, tuple(t.shape), ", ".join("*" if e is None else str(e) for e in shape)))
    raise ValueError("%s must be contiguous" % name)


def _check_cache(k_cache, v_cache, k_scale, v_scale, num_kv_heads, page_size, head_dim, kv_format,
                 device):
    """K/V caches [num_pages, Hkv, P, D] (bf16, or e4m3fn bytes as uint8 or float8_e4m3fn)
    and, for fp8, fp32 scales [num_pages, Hkv]. Returns num_pages."""
    import torch
    fp8 = kv_format in ("fp8", KV_FP8_E4M3FN)
    kinds = (torch.uint8, torch.float8_e4m3fn) if fp8 else (torch.bfloat16,)
    _check_tensor(k_cache, "k_cache", kinds, (None, num_kv_heads, page_size, head_dim), device)
    n = int(k_cache.shape[0])
    _check_tensor(v_cache, "v_cache", kinds, (n, num_kv_heads, page_size, head_dim), device)
    if fp8:
        for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            _check_tensor(t, name, (torch.float32,), (n, num_kv_heads), device)
    return n


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------------
# C ABI, one wrapper per entry point


def pkv_abi_version():
    return _lib.pkv_abi_version()


def pkv_status_string(status):
    return _status_text(status)


def pkv_last_error():
    return _lib.pkv_last_error().decode()


def pkv_plan_query(seq_lens_h, q_len, num_q_heads, num_kv_heads, head_dim, page_size, kv_format,
                   tile_tokens, num_workers):
    """Returns (tile_tokens, num_items, num_partials)."""
    sl, slp = _i32(seq_lens_h)
    T = ctypes.c_int32()
    N = ctypes.c_int64()
    NP = ctypes.c_int64()
    _check(_lib.pkv_plan_query(len(sl), slp, q_len, num_q_heads, num_kv_heads, head_dim, page_size,
                               KV_FORMATS.get(kv_format, kv_format), tile_tokens, num_workers,
                               ctypes.byref(T), ctypes.byref(N), ctypes.byref(NP)), "pkv_plan_query")
    return T.value, N.value, NP.value


def pkv_plan(seq_lens_h, q_len, num_kv_heads, tile_tokens, num_workers, num_items=None, out=None):
    """Build the plan. Returns (items [N,4], worker_offsets [W+1], req_tile_base [B+1]) as
    int32 numpy arrays; with ``out`` = (items, offsets, rtb) writes into those arrays."""
    sl, slp = _i32(seq_lens_h)
    B = len(sl)
    if out is None:
        if num_items is None:
            num_items = sum((int(L) + tile_tokens - 1) // tile_tokens for L in sl) * num_kv_heads
        out = (np.empty((num_items, 4), np.int32), np.empty(num_workers + 1, np.int32),
               np.empty(B + 1, np.int32))
    items, offs, rtb = out
    for a in out:
        assert a.dtype == np.int32 and a.flags.c_contiguous
    _check(_lib.pkv_plan(B, slp, q_len, num_kv_heads, tile_tokens, num_workers,
                         items.ctypes.data_as(_i32p), offs.ctypes.data_as(_i32p),
                         rtb.ctypes.data_as(_i32p)), "pkv_plan")
    return items, offs, rtb


def pkv_default_num_workers(device=0, kv_format="bf16", head_dim=128):
    out = ctypes.c_int()
    _check(_lib.pkv_default_num_workers(device, KV_FORMATS.get(kv_format, kv_format), head_dim,
                                        ctypes.byref(out)), "pkv_default_num_workers")
    return out.value


def pkv_workspace_bytes(num_partials, rows_per_partial, head_dim):
    out = ctypes.c_size_t()
    _check(_lib.pkv_workspace_bytes(num_partials, rows_per_partial, head_dim, ctypes.byref(out)),
           "pkv_workspace_bytes")
    return out.value


def _decode_args(*, q, k_cache, v_cache, block_table, seq_lens, items, worker_offsets,
                 req_tile_base, workspace, workspace_bytes, num_items, num_partials, num_pages,
                 batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride,
                 kv_format, tile_tokens, num_workers, scale, k_scale=None, v_scale=None,
                 tile_tokens_dev=None, request_split=1, direct_out=None, direct_lse_out=None):
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.q, a.k_cache, a.v_cache = _ptr(q, "q"), _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache")
    a.k_scale, a.v_scale = _ptr(k_scale, "k_scale"), _ptr(v_scale, "v_scale")
    a.block_table, a.seq_lens = _ptr(block_table, "block_table"), _ptr(seq_lens, "seq_lens")
    a.items = _ptr(items, "items")
    a.worker_offsets = _ptr(worker_offsets, "worker_offsets")
    a.req_tile_base = _ptr(req_tile_base, "req_tile_base")
    a.workspace, a.workspace_bytes = _ptr(workspace, "workspace"), workspace_bytes
    a.num_items, a.num_partials, a.num_pages = num_items, num_partials, num_pages
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads = batch, q_len, num_q_heads, num_kv_heads
    a.head_dim, a.page_size, a.bt_stride = head_dim, page_size, bt_stride
    a.kv_format = KV_FORMATS.get(kv_format, kv_format)
    a.tile_tokens, a.num_workers, a.scale = tile_tokens, num_workers, scale
    a.tile_tokens_dev = _ptr(tile_tokens_dev, "tile_tokens_dev")
    a.request_split = request_split
    a.out = _ptr(direct_out, "direct_out")
    a.lse_out = _ptr(direct_lse_out, "direct_lse_out")
    return a


def pkv_decode_partial(*, stream=None, **kw):
    """Enqueue the split-KV partial kernel. Device arguments are tensors or raw addresses
    (keywords as the fields of pkv_decode_args; its optional out / lse_out are
    direct_out / direct_lse_out here)."""
    a = _decode_args(**kw)
    _check(_lib.pkv_decode_partial(ctypes.byref(a), _stream_handle(stream)), "pkv_decode_partial")


PKV_NOALLOC_SCRATCH_BYTES = 32 << 20


def pkv_decode_noalloc(*, out, lse_out=None, stream=None, workspace=None, workspace_bytes=0, **kw):
    """Enqueue a whole decode step (partials + combine) whose partials live in the
    library's own device array (no workspace, no allocation); keywords as for
    pkv_decode_partial, plus out / lse_out as for pkv_combine."""
    a = _decode_args(workspace=workspace, workspace_bytes=workspace_bytes, **kw)
    _check(_lib.pkv_decode_noalloc(ctypes.byref(a), _ptr(out, "out"), _ptr(lse_out, "lse_out"),
                                   _stream_handle(stream)), "pkv_decode_noalloc")


def pkv_plan_device_scratch_bytes(batch, num_kv_heads, page_size, kv_format, tile_tokens,
                                  num_workers, max_items):
    out = ctypes.c_size_t()
    _check(_lib.pkv_plan_device_scratch_bytes(batch, num_kv_heads, page_size,
                                              KV_FORMATS.get(kv_format, kv_format), tile_tokens,
                                              num_workers, max_items, ctypes.byref(out)),
           "pkv_plan_device_scratch_bytes")
    return out.value


def pkv_plan_device(*, seq_lens, batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size,
                    kv_format, tile_tokens, num_workers, max_items, items, worker_offsets,
                    req_tile_base, info, scratch, scratch_bytes, stream=None):
    """Enqueue the device-side planner (same work list as pkv_plan, built on the GPU)."""
    _check(_lib.pkv_plan_device(_ptr(seq_lens, "seq_lens"), batch, q_len, num_q_heads, num_kv_heads,
                                head_dim, page_size, KV_FORMATS.get(kv_format, kv_format),
                                tile_tokens, num_workers, max_items, _ptr(items, "items"),
                                _ptr(worker_offsets, "worker_offsets"),
                                _ptr(req_tile_base, "req_tile_base"), _ptr(info, "info"),
                                _ptr(scratch, "scratch"), scratch_bytes, _stream_handle(stream)),
           "pkv_plan_device")


def pkv_combine(*, workspace, workspace_bytes, num_partials, req_tile_base, batch, q_len,
                num_q_heads, num_kv_heads, head_dim, out, lse_out=None, stream=None):
    """Enqueue the log-sum-exp combine kernel."""
    _check(_lib.pkv_combine(_ptr(workspace, "workspace"), workspace_bytes, num_partials,
                            _ptr(req_tile_base, "req_tile_base"), batch, q_len, num_q_heads,
                            num_kv_heads, head_dim, _ptr(out, "out"), _ptr(lse_out, "lse_out"),
                            _stream_handle(stream)), "pkv_combine")


def pkv_combine_split(*, workspace, workspace_bytes, num_partials, req_tile_base, batch, q_len,
                      num_q_heads, num_kv_heads, head_dim, request_split, out, lse_out=None,
                      stream=None):
    """Enqueue the combine for a work list whose requests are split in parts."""
    _check(_lib.pkv_combine_split(_ptr(workspace, "workspace"), workspace_bytes, num_partials,
                                  _ptr(req_tile_base, "req_tile_base"), batch, q_len, num_q_heads,
                                  num_kv_heads, head_dim, request_split, _ptr(out, "out"),
                                  _ptr(lse_out, "lse_out"), _stream_handle(stream)),
           "pkv_combine_split")


def pkv_block_sparse_compact(*, block_table, seq_lens, block_mask, batch, num_kv_heads, q_len,
                             page_size, bt_stride, mask_stride, num_pages, bt_out, seq_lens_out,
                             stream=None):
    """Enqueue the block-mask compaction into a one-kv-head problem (see include/pkv.h)."""
    _check(_lib.pkv_block_sparse_compact(_ptr(block_table, "block_table"), _ptr(seq_lens, "seq_lens"),
                                         _ptr(block_mask, "block_mask"), batch, num_kv_heads, q_len,
                                         page_size, bt_stride, mask_stride, num_pages,
                                         _ptr(bt_out, "bt_out"), _ptr(seq_lens_out, "seq_lens_out"),
                                         _stream_handle(stream)),
           "pkv_block_sparse_compact")


def pkv_block_sparse_lengths(seq_lens_h, block_mask_h, num_kv_heads, q_len, page_size):
    """Host lengths of the compacted one-kv-head problem: int32 [B * num_kv_heads]."""
    sl, slp = _i32(seq_lens_h)
    m = np.ascontiguousarray(block_mask_h, dtype=np.uint8)
    B = len(sl)
    out = np.empty(B * num_kv_heads, np.int32)
    _check(_lib.pkv_block_sparse_lengths(B, slp, m.ctypes.data, num_kv_heads, q_len, page_size,
                                         m.shape[-1], out.ctypes.data_as(_i32p)),
           "pkv_block_sparse_lengths")
    return out


def pkv_kv_append(*, k_new, v_new, k_cache, v_cache, block_table, seq_lens, num_pages, batch,
                  q_len, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride, kv_format,
                  q=None, q_out=None, rope_cos=None, rope_sin=None, max_pos=0, k_scale=None,
                  v_scale=None, stream=None):
    """Enqueue the fused KV append (rotary embedding, paged write, fp8 quantise-on-write)."""
    a = KvAppendArgs()
    a.struct_size = ctypes.sizeof(KvAppendArgs)
    a.k_new, a.v_new = _ptr(k_new, "k_new"), _ptr(v_new, "v_new")
    a.q, a.q_out = _ptr(q, "q"), _ptr(q_out, "q_out")
    a.rope_cos, a.rope_sin = _ptr(rope_cos, "rope_cos"), _ptr(rope_sin, "rope_sin")
    a.k_cache, a.v_cache = _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache")
    a.k_scale, a.v_scale = _ptr(k_scale, "k_scale"), _ptr(v_scale, "v_scale")
    a.block_table, a.seq_lens = _ptr(block_table, "block_table"), _ptr(seq_lens, "seq_lens")
    a.num_pages, a.batch, a.q_len = num_pages, batch, q_len
    a.num_q_heads, a.num_kv_heads, a.head_dim = num_q_heads, num_kv_heads, head_dim
    a.page_size, a.bt_stride = page_size, bt_stride
    a.kv_format = KV_FORMATS.get(kv_format, kv_format)
    a.max_pos = max_pos
    _check(_lib.pkv_kv_append(ctypes.byref(a), _stream_handle(stream)), "pkv_kv_append")


def pkv_prefill_plan_size(q_lens_h, num_q_heads, num_kv_heads):
    ql, qlp = _i32(q_lens_h)
    n = ctypes.c_int64()
    _check(_lib.pkv_prefill_plan_size(len(ql), qlp, num_q_heads, num_kv_heads, ctypes.byref(n)),
           "pkv_prefill_plan_size")
    return n.value


def pkv_prefill_plan(q_lens_h, kv_lens_h, num_q_heads, num_kv_heads):
    """Prefill work items, int32 [N, 4] rows (b, g, head group, first token), heaviest
    first."""
    ql, qlp = _i32(q_lens_h)
    kl, klp = _i32(kv_lens_h)
    n = pkv_prefill_plan_size(ql, num_q_heads, num_kv_heads)
    items = np.empty((n, 4), np.int32)
    _check(_lib.pkv_prefill_plan(len(ql), qlp, klp, num_q_heads, num_kv_heads,
                                 items.ctypes.data_as(_i32p)), "pkv_prefill_plan")
    return items


def pkv_prefill(*, q, cu_q, kv_lens, block_table, items, num_items, k_cache, v_cache, out,
                num_pages, batch, num_q_heads, num_kv_heads, head_dim, page_size, bt_stride,
                kv_format, scale, k_scale=None, v_scale=None, lse=None, stream=None):
    """Enqueue variable-length causal prefill over the paged cache."""
    a = PrefillArgs()
    a.struct_size = ctypes.sizeof(PrefillArgs)
    a.q, a.cu_q, a.kv_lens = _ptr(q, "q"), _ptr(cu_q, "cu_q"), _ptr(kv_lens, "kv_lens")
    a.block_table, a.items = _ptr(block_table, "block_table"), _ptr(items, "items")
    a.k_cache, a.v_cache = _ptr(k_cache, "k_cache"), _ptr(v_cache, "v_cache")
    a.k_scale, a.v_scale = _ptr(k_scale, "k_scale"), _ptr(v_scale, "v_scale")
    a.out, a.lse = _ptr(out, "out"), _ptr(lse, "lse")
    a.num_items, a.num_pages, a.batch = num_items, num_pages, batch
    a.num_q_heads, a.num_kv_heads, a.head_dim = num_q_heads, num_kv_heads, head_dim
    a.page_size, a.bt_stride = page_size, bt_stride
    a.kv_format = KV_FORMATS.get(kv_format, kv_format)
    a.scale = scale
    _check(_lib.pkv_prefill(ctypes.byref(a), _stream_handle(stream)), "pkv_prefill")


class PagedPrefill:
    """Variable-length causal prefill over the paged cache: host tile plan (copied to the
    device on the current stream) + the prefill kernel."""

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, page_size, kv_format="bf16",
                 device=None):
        import torch
        self.torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.head_dim, self.page_size, self.kv_format = head_dim, page_size, kv_format
        self.last_items = None

    def plan(self, q_lens_h, kv_lens_h):
        items = pkv_prefill_plan(q_lens_h, kv_lens_h, self.num_q_heads, self.num_kv_heads)
        self.last_items = items
        return self.torch.from_numpy(items).to(self.device, non_blocking=False)

    def __call__(self, q, cu_q, kv_lens, block_table, q_lens_h, kv_lens_h, scale, *, k_cache,
                 v_cache, k_scale=None, v_scale=None, out=None, lse=None, items=None, stream=None):
        """q bf16 [total, Hq, D]; cu_q / kv_lens device int32; q_lens_h / kv_lens_h host
        copies (for the plan). ``items``: a device plan from ``plan`` to reuse."""
        torch = self.torch
        Hq, D, dev = self.num_q_heads, self.head_dim, self.device
        _check_tensor(cu_q, "cu_q", (torch.int32,), (None,), dev)
        B = int(cu_q.shape[0]) - 1
        if B < 0:
            raise ValueError("cu_q needs batch + 1 entries")
        _check_tensor(q, "q", (torch.bfloat16,), (None, Hq, D), dev)
        _check_tensor(kv_lens, "kv_lens", (torch.int32,), (B,), dev)
        _check_tensor(block_table, "block_table", (torch.int32,), (B, None), dev)
        _check_cache(k_cache, v_cache, k_scale, v_scale, self.num_kv_heads, self.page_size, D,
                     self.kv_format, dev)
        if len(q_lens_h) != B or len(kv_lens_h) != B:
            raise ValueError("q_lens_h and kv_lens_h need one entry per request")
        if out is not None:
            _check_tensor(out, "out", (torch.bfloat16,), tuple(q.shape), dev)
        if lse is not None:
            _check_tensor(lse, "lse", (torch.float32,), (int(q.shape[0]), Hq), dev)
        if items is None:
            items = self.plan(q_lens_h, kv_lens_h)
        else:
            _check_tensor(items, "items", (torch.int32,), (None, 4), dev)
        if out is None:
            out = torch.empty_like(q)
        pkv_prefill(q=q, cu_q=cu_q, kv_lens=kv_lens, block_table=block_table, items=items,
                    num_items=items.shape[0], k_cache=k_cache, v_cache=v_cache, out=out,
                    num_pages=k_cache.shape[0], batch=int(cu_q.shape[0]) - 1,
                    num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads,
                    head_dim=self.head_dim, page_size=self.page_size,
                    bt_stride=block_table.shape[1], kv_format=self.kv_format, scale=scale,
                    k_scale=k_scale, v_scale=v_scale, lse=lse, stream=stream)
        return out


# ---------------------------------------------------------------------------------
# Per-step runner


_HIP_HOST_MALLOC_MAPPED = 0x2
_HIP_HOST_MALLOC_COHERENT = 0x40000000


def _hip_runtime():
    """The HIP runtime torch has loaded (dlopen by soname returns the loaded copy): the
    ROCm 7 soname first, then older and unversioned ones."""
    err = None
    for name in ("libamdhip64.so.7", "libamdhip64.so.6", "libamdhip64.so"):
        try:
            return ctypes.CDLL(name)
        except OSError as e:
            err = e
    raise ImportError("no HIP runtime (libamdhip64) could be loaded: %s" % err)


class HostPlanBuffer:
    """Pinned, device-mapped, coherent host memory for one step's plan.

    The kernels read the plan straight from here (zero-copy), so the step needs no
    host-to-device copy. Coherent memory is not cached by the GPU, so every launch
    sees what the host wrote before it."""

    _hip = None

    def __init__(self, nbytes):
        if HostPlanBuffer._hip is None:
            hip = _hip_runtime()
            hip.hipHostMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t, ctypes.c_uint]
            hip.hipHostMalloc.restype = ctypes.c_int
            hip.hipHostFree.argtypes = [ctypes.c_void_p]
            hip.hipHostFree.restype = ctypes.c_int
            HostPlanBuffer._hip = hip
        self._ptr = ctypes.c_void_p()
        rc = HostPlanBuffer._hip.hipHostMalloc(ctypes.byref(self._ptr), nbytes,
                                               _HIP_HOST_MALLOC_MAPPED | _HIP_HOST_MALLOC_COHERENT)
        if rc != 0 or not self._ptr.value:
            raise RuntimeError("hipHostMalloc(%d bytes, coherent) failed: %d" % (nbytes, rc))
        self.nbytes = nbytes
        self.addr = self._ptr.value
        self.array = np.ctypeslib.as_array((ctypes.c_int32 * (nbytes // 4)).from_address(self.addr))

    def free(self):
        hip = type(self)._hip
        if hip is not None and self._ptr is not None and self._ptr.value:
            hip.hipHostFree(self._ptr)
        self._ptr = None


class PagedDecode:
    """One decode step = plan + decode_partial + combine, enqueued on the current torch
    stream with no host synchronisation.

    Host plan (default): the plan is written into a ring of coherent pinned buffers
    that the kernels read directly (no host-to-device copy on the step's critical
    path). A buffer is rewritten only after the kernels of the step that last read it
    have completed (an event per buffer).
    Device plan (``device_plan=True``): ``pkv_plan_device`` builds the same plan on
    the GPU from device seq_lens, so the step needs no host lengths and can be
    captured in a graph.
    Block-sparse decode: pass ``block_mask`` (device uint8 [B, Hkv, >= bt_stride]); the
    step compacts it (``pkv_block_sparse_compact``) into a one-kv-head problem of
    B * Hkv requests and runs the same kernels on it. It is planned on the host when the
    host copy ``block_mask_h`` is given (for the lengths), else on the device.
    The workspace and device buffers grow on demand and are kept, so at a fixed shape
    no allocation happens after the first steps."""

    def __init__(self, *, num_q_heads, num_kv_heads, head_dim, page_size, kv_format="bf16",
                 q_len=1, tile_tokens=0, num_workers=0, device=None, slots=3,
                 device_plan=False, max_items=0):
        import torch
        self.torch = torch
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.head_dim, self.page_size, self.kv_format = head_dim, page_size, kv_format
        self.q_len, self.tile_tokens = q_len, tile_tokens
        self.rows = (num_q_heads // num_kv_heads) * q_len
        self.num_workers = num_workers or pkv_default_num_workers(self.device.index, kv_format, head_dim)
        self._bufs = [None] * slots
        self._consumed = [None] * slots    # event on the compute stream: kernels reading slot done
        self._slot = 0
        self._workspace = None
        self.last_plan = None
        # Device-built plan (pkv_plan_device): no host work per step, so the step can
        # be captured in a graph. max_items is the plan's item capacity (0 = a bound
        # derived from the block table's width).
        self.device_plan = device_plan
        self.max_items = max_items
        self._dev = None
        self._sparse = None
        self._fmt = KV_FORMATS.get(kv_format, kv_format)
        T, N, NP = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        self._query_out = (T, N, NP, ctypes.byref(T), ctypes.byref(N), ctypes.byref(NP))

    def close(self):
        """Free the plan buffers (after the kernels that read them have completed)."""
        for k, buf in enumerate(getattr(self, "_bufs", [])):
            if buf is not None:
                ev = self._consumed[k]
                if ev is not None:
                    ev.synchronize()
                buf.free()
                self._bufs[k] = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001  (interpreter shutdown: the process releases it)
            pass

    def plan(self, seq_lens_h, num_q_heads=None, num_kv_heads=None):
        """Host plan into the next plan buffer; returns a dict describing it. The head
        counts default to the runner's (block-sparse steps plan a one-kv-head problem).
        The buffer holds seq_lens [B], then items [N][4], worker offsets [W+1] and the
        tile prefix [B+1], each 16-byte aligned; the planner reads and writes it by
        address (numpy's ctypes conversions would cost several microseconds each)."""
        Hq = num_q_heads or self.num_q_heads
        Hkv = num_kv_heads or self.num_kv_heads
        sl = np.ascontiguousarray(seq_lens_h, dtype=np.int32)
        W, B = self.num_workers, len(sl)
        n_items = _round4(B)
        k = self._slot
        self._slot = (k + 1) % len(self._bufs)
        if self._consumed[k] is not None:
            self._consumed[k].synchronize()        # the kernels that last read this buffer are done
        buf = self._bufs[k]
        if buf is None or buf.nbytes < 4 * (n_items + 4096):
            buf = self._grow(k, 4 * (n_items + 4096))
        buf.array[:B] = sl
        a = buf.addr
        q = self._query_out
        _check(_lib.pkv_plan_query(B, a, self.q_len, Hq, Hkv, self.head_dim, self.page_size,
                                   self._fmt, self.tile_tokens, W, q[3], q[4], q[5]), "pkv_plan_query")
        T, N, NP = q[0].value, q[1].value, q[2].value
        n_off = n_items + 4 * N
        n_rtb = n_off + _round4(W + 1)
        total = n_rtb + _round4(B + 1)
        if buf.nbytes < 4 * total:
            buf = self._grow(k, 4 * total)
            buf.array[:B] = sl
            a = buf.addr
        _check(_lib.pkv_plan(B, a, self.q_len, Hkv, T, W, a + 4 * n_items, a + 4 * n_off,
                             a + 4 * n_rtb), "pkv_plan")
        p = dict(T=T, N=N, NP=NP, W=W, B=B, slot=k, items=a + 4 * n_items,
                 worker_offsets=a + 4 * n_off, req_tile_base=a + 4 * n_rtb, seq_lens=a)
        self.last_plan = p
        return p

    def _grow(self, k, nbytes):
        """Replace plan buffer k (idle: its kernels have completed) by one of nbytes."""
        if self._bufs[k] is not None:
            self._bufs[k].free()
        self._bufs[k] = HostPlanBuffer(nbytes)
        return self._bufs[k]

    def default_capacity(self, batch, bt_stride, num_kv_heads=None):
        """Item capacity of a device-built plan. For a fixed tile: the most items any
        lengths up to bt_stride pages can need. For the automatic tile: room for the
        largest candidate tile (65536) at any such lengths, plus 8 items per worker."""
        max_len = bt_stride * self.page_size
        H = num_kv_heads or self.num_kv_heads
        if self.tile_tokens:
            return batch * H * (-(-max_len // self.tile_tokens))
        return 8 * self.num_workers + batch * H * (1 + -(-max_len // 65536))

    def device_buffers(self, batch, bt_stride, num_kv_heads=None):
        """The device plan's buffers for a batch size (allocated on first use)."""
        torch = self.torch
        H = num_kv_heads or self.num_kv_heads
        cap = self.max_items or self.default_capacity(batch, bt_stride, H)
        key = (batch, H, cap)
        if self._dev is None or self._dev["key"] != key:
            nscratch = pkv_plan_device_scratch_bytes(batch, H, self.page_size, self.kv_format,
                                                     self.tile_tokens, self.num_workers, cap)
            i32 = dict(dtype=torch.int32, device=self.device)
            self._dev = dict(key=key, cap=cap, items=torch.empty((max(cap, 1), 4), **i32),
                             offsets=torch.empty(self.num_workers + 1, **i32),
                             rtb=torch.empty(batch + 1, **i32), info=torch.zeros(4, **i32),
                             scratch=torch.empty(nscratch, dtype=torch.uint8, device=self.device),
                             scratch_bytes=nscratch)
        return self._dev

    def sparse_buffers(self, batch, bt_stride):
        """Compacted block table [B * Hkv, bt_stride] and lengths [B * Hkv]."""
        key = (batch, bt_stride)
        if self._sparse is None or self._sparse["key"] != key:
            i32 = dict(dtype=self.torch.int32, device=self.device)
            n = batch * self.num_kv_heads
            self._sparse = dict(key=key, bt=self.torch.empty((max(n, 1), bt_stride), **i32),
                                sl=self.torch.empty(max(n, 1), **i32))
        return self._sparse

    def plan_info(self):
        """Status, tile, item count and most items per worker of the last device plan
        (synchronises with the device)."""
        if self._dev is None:
            return None
        st, T, N, mx = (int(x) for x in self._dev["info"].cpu())
        return dict(status=st, T=T, N=N, max_items_per_worker=mx, capacity=self._dev["cap"])

    def append(self, k_new, v_new, k_cache, v_cache, block_table, seq_lens, *, q=None, q_out=None,
               rope_cos=None, rope_sin=None, k_scale=None, v_scale=None, stream=None):
        """Enqueue the fused KV append for this runner's shapes: the step's new k/v rows
        (bf16 [B, Tq, Hkv, D]) into the paged cache, optionally rotating q into q_out and
        the k rows by the tables (fp32 [max_pos, D/2]); fp8 pages are quantised on write."""
        torch, dev = self.torch, self.device
        Tq, Hq, Hkv, D = self.q_len, self.num_q_heads, self.num_kv_heads, self.head_dim
        _check_tensor(seq_lens, "seq_lens", (torch.int32,), (None,), dev)
        B = int(seq_lens.shape[0])
        for t, name in ((k_new, "k_new"), (v_new, "v_new")):
            _check_tensor(t, name, (torch.bfloat16,), (B, Tq, Hkv, D), dev)
        _check_tensor(block_table, "block_table", (torch.int32,), (B, None), dev)
        _check_cache(k_cache, v_cache, k_scale, v_scale, Hkv, self.page_size, D, self.kv_format, dev)
        if (q is None) != (q_out is None) or (rope_cos is None) != (rope_sin is None):
            raise ValueError("q and q_out, and rope_cos and rope_sin, come in pairs")
        for t, name in ((q, "q"), (q_out, "q_out")):
            if t is not None:
                _check_tensor(t, name, (torch.bfloat16,), (B, Tq, Hq, D), dev)
        for t, name in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
            if t is not None:
                _check_tensor(t, name, (torch.float32,), (int(rope_cos.shape[0]), D // 2), dev)
        pkv_kv_append(k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                      block_table=block_table, seq_lens=seq_lens, num_pages=k_cache.shape[0],
                      batch=int(seq_lens.shape[0]), q_len=self.q_len, num_q_heads=self.num_q_heads,
                      num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                      page_size=self.page_size, bt_stride=block_table.shape[1],
                      kv_format=self.kv_format, q=q, q_out=q_out, rope_cos=rope_cos,
                      rope_sin=rope_sin, max_pos=0 if rope_cos is None else rope_cos.shape[0],
                      k_scale=k_scale, v_scale=v_scale, stream=stream)

    def workspace(self, num_partials):
        nbytes = pkv_workspace_bytes(max(num_partials, 1), self.rows, self.head_dim)
        if self._workspace is None or self._workspace.numel() < nbytes:
            self.torch.cuda.synchronize(self.device)
            self._workspace = self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.device)
        return self._workspace, nbytes

    def __call__(self, q, k_cache, v_cache, block_table, seq_lens_h, scale, *, k_scale=None,
                 v_scale=None, seq_lens=None, out=None, lse_out=None, stream=None,
                 partial_events=None, block_mask=None, block_mask_h=None):
        """Run one decode step. ``seq_lens_h`` (host ints) drives a host plan; ``seq_lens``
        (device int32) defaults to the copy written next to it and is required for a
        device plan and for block-sparse steps. ``block_mask`` (device uint8 [B, Hkv,
        mask_stride]) makes the step block-sparse; ``block_mask_h`` is its host copy, which
        lets it be planned on the host (without it the plan is built on the device). ``partial_events``: two torch.cuda.Events recorded
        around the decode_partial launch (for timing)."""
        if stream is not None:
            with self.torch.cuda.stream(stream):
                return self(q, k_cache, v_cache, block_table, seq_lens_h, scale, k_scale=k_scale,
                            v_scale=v_scale, seq_lens=seq_lens, out=out, lse_out=lse_out,
                            partial_events=partial_events, block_mask=block_mask,
                            block_mask_h=block_mask_h)
        torch = self.torch
        Hkv, G = self.num_kv_heads, self.num_q_heads // self.num_kv_heads
        Tq, Hq, D, dev = self.q_len, self.num_q_heads, self.head_dim, self.device
        if seq_lens is not None:
            _check_tensor(seq_lens, "seq_lens", (torch.int32,), (None,), dev)
        B = int(seq_lens.shape[0]) if seq_lens is not None else len(seq_lens_h)
        if seq_lens_h is not None and len(seq_lens_h) != B:
            raise ValueError("seq_lens_h has %d entries, seq_lens %d" % (len(seq_lens_h), B))
        _check_tensor(q, "q", (torch.bfloat16,), (B, Tq, Hq, D), dev)
        _check_tensor(block_table, "block_table", (torch.int32,), (B, None), dev)
        _check_cache(k_cache, v_cache, k_scale, v_scale, Hkv, self.page_size, D, self.kv_format, dev)
        if out is not None:
            _check_tensor(out, "out", (torch.bfloat16,), (B, Tq, Hq, D), dev)
        if lse_out is not None:
            _check_tensor(lse_out, "lse_out", (torch.float32,), (B, Tq, Hq), dev)
        if block_mask is not None:
            _check_tensor(block_mask, "block_mask", (torch.uint8,), (B, Hkv, None), dev)
            if block_mask_h is not None and tuple(np.shape(block_mask_h)) != tuple(block_mask.shape):
                raise ValueError("block_mask_h must have block_mask's shape")
        bt_stride = block_table.shape[1]
        sh = torch.cuda.current_stream(dev).cuda_stream   # one lookup for every launch below
        if block_mask is not None:
            # The one-kv-head problem: B * Hkv requests over the cache viewed as
            # [num_pages * Hkv, 1, P, D].
            if seq_lens is None or not getattr(seq_lens, "is_cuda", False):
                raise ValueError("a block-sparse step needs seq_lens as a CUDA int32 tensor")
            sp = self.sparse_buffers(B, bt_stride)
            mask_stride = block_mask.shape[-1]
            pkv_block_sparse_compact(block_table=block_table, seq_lens=seq_lens, block_mask=block_mask,
                                     batch=B, num_kv_heads=Hkv, q_len=self.q_len,
                                     page_size=self.page_size, bt_stride=bt_stride,
                                     mask_stride=mask_stride, num_pages=k_cache.shape[0],
                                     bt_out=sp["bt"], seq_lens_out=sp["sl"], stream=sh)
            prob = dict(batch=B * Hkv, Hq=G, Hkv=1, split=Hkv, bt=sp["bt"], sl=sp["sl"],
                        num_pages=k_cache.shape[0] * Hkv)
            use_device_plan = self.device_plan or block_mask_h is None
            if not use_device_plan:
                lengths_h = pkv_block_sparse_lengths(seq_lens_h, block_mask_h, Hkv, self.q_len,
                                                     self.page_size)
        else:
            prob = dict(batch=B, Hq=self.num_q_heads, Hkv=Hkv, split=1, bt=block_table, sl=seq_lens,
                        num_pages=k_cache.shape[0])
            lengths_h = seq_lens_h
            use_device_plan = self.device_plan
        tile_dev = None
        if use_device_plan:
            if prob["sl"] is None or not getattr(prob["sl"], "is_cuda", False):
                raise ValueError("a device-built plan needs seq_lens as a CUDA int32 tensor")
            d = self.device_buffers(prob["batch"], bt_stride, prob["Hkv"])
            pkv_plan_device(seq_lens=prob["sl"], batch=prob["batch"], q_len=self.q_len,
                            num_q_heads=prob["Hq"], num_kv_heads=prob["Hkv"], head_dim=self.head_dim,
                            page_size=self.page_size, kv_format=self.kv_format,
                            tile_tokens=self.tile_tokens, num_workers=self.num_workers,
                            max_items=d["cap"], items=d["items"], worker_offsets=d["offsets"],
                            req_tile_base=d["rtb"], info=d["info"], scratch=d["scratch"],
                            scratch_bytes=d["scratch_bytes"], stream=sh)
            p = dict(T=self.tile_tokens, N=d["cap"], NP=d["cap"], W=self.num_workers, slot=None,
                     items=d["items"], worker_offsets=d["offsets"], req_tile_base=d["rtb"])
            tile_dev = d["info"][1:]
            sl_dev = prob["sl"]
        else:
            p = self.plan(lengths_h, prob["Hq"], prob["Hkv"])
            sl_dev = prob["sl"] if prob["sl"] is not None else p["seq_lens"]
        ws, ws_bytes = self.workspace(p["NP"])
        if out is None:
            out = torch.empty((B, self.q_len, self.num_q_heads, self.head_dim), dtype=torch.bfloat16,
                              device=self.device)
        if partial_events is not None:
            partial_events[0].record()
        pkv_decode_partial(q=q, k_cache=k_cache, v_cache=v_cache, block_table=prob["bt"],
                           seq_lens=sl_dev, items=p["items"], worker_offsets=p["worker_offsets"],
                           req_tile_base=p["req_tile_base"], workspace=ws, workspace_bytes=ws_bytes,
                           num_items=p["N"], num_partials=p["NP"], num_pages=prob["num_pages"],
                           batch=prob["batch"], q_len=self.q_len, num_q_heads=prob["Hq"],
                           num_kv_heads=prob["Hkv"], head_dim=self.head_dim,
                           page_size=self.page_size, bt_stride=bt_stride,
                           kv_format=self.kv_format, tile_tokens=p["T"], num_workers=p["W"],
                           scale=scale, k_scale=k_scale, v_scale=v_scale, tile_tokens_dev=tile_dev,
                           request_split=prob["split"],
                           direct_out=out if prob["split"] == 1 else None,
                           direct_lse_out=lse_out if prob["split"] == 1 else None, stream=sh)
        if partial_events is not None:
            partial_events[1].record()
        # A host plan with one tile per request leaves nothing to merge: decode_partial
        # has already written every final row (the combine would rewrite the same bits).
        single = (not use_device_plan and prob["split"] == 1
                  and p["N"] == prob["batch"] * prob["Hkv"])
        if not single:
            pkv_combine_split(workspace=ws, workspace_bytes=ws_bytes, num_partials=p["NP"],
                              req_tile_base=p["req_tile_base"], batch=prob["batch"], q_len=self.q_len,
                              num_q_heads=prob["Hq"], num_kv_heads=prob["Hkv"],
                              head_dim=self.head_dim, request_split=prob["split"], out=out,
                              lse_out=lse_out, stream=sh)
        k = p["slot"]
        if k is not None:
            if self._consumed[k] is None:
                self._consumed[k] = torch.cuda.Event()
            self._consumed[k].record()
        return out


def _round4(x):
    return (x + 3) // 4 * 4
