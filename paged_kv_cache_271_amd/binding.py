"""Thin ctypes binding of libpagedkv (argument marshalling only).

Functions carry the C names.  Device buffers are torch tensors on a HIP
device; host arrays are numpy int32 arrays.  Every computation runs in the
library's HIP kernels or in its C++ host code: there is no Python fallback,
and a missing library raises at load time.
"""

import ctypes
import os

import numpy as np

from .build import LIB_PATH

KV_F32, KV_BF16, KV_FP8_E4M3, KV_INT8 = 0, 1, 2, 3
STATUS = {0: "KV_OK", -1: "KV_E_INVALID", -2: "KV_E_UNSUPPORTED", -3: "KV_E_NO_BLOCKS",
          -4: "KV_E_BAD_BLOCK", -5: "KV_E_SHARED", -6: "KV_E_WORKSPACE", -7: "KV_E_HIP"}
DTYPE_NAMES = {"f32": KV_F32, "bf16": KV_BF16, "fp8": KV_FP8_E4M3, "int8": KV_INT8}
BLOCK_SIZE = 16

# every function include/*.h declares: name -> (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


class KvPoolDesc(ctypes.Structure):
    _fields_ = [("num_layers", _I32), ("num_blocks", _I32), ("block_size", _I32),
                ("num_kv_heads", _I32), ("head_dim", _I32), ("cache_dtype", _I32)]


_PDESC = ctypes.POINTER(KvPoolDesc)
SIGNATURES = {
    "kv_bytes_per_token": (_I64, [_PDESC]),
    "kv_blocks_for_tokens": (_I32, [_I32, _I32]),
    "kv_pool_buffer_bytes": (ctypes.c_int, [_PDESC, _PI64, _PI64]),
    "kv_pool_create": (ctypes.c_int, [_PDESC, _P, _P, _P, _P, _PI32, ctypes.POINTER(_P)]),
    "kv_pool_destroy": (ctypes.c_int, [_P]),
    "kv_block_alloc": (ctypes.c_int, [_P, _PI32]),
    "kv_block_retain": (ctypes.c_int, [_P, _I32]),
    "kv_block_release": (ctypes.c_int, [_P, _I32]),
    "kv_block_retain_n": (ctypes.c_int, [_P, _PI32, _I32]),
    "kv_block_release_n": (ctypes.c_int, [_P, _PI32, _I32]),
    "kv_block_refcount": (ctypes.c_int, [_P, _I32, _PI32]),
    "kv_num_free_blocks": (ctypes.c_int, [_P, _PI32]),
    "kv_num_shared_blocks": (ctypes.c_int, [_P, _PI32]),
    "kv_slot_mapping": (ctypes.c_int, [_P, _PI32, _I32, _PI32, _I32, _PI32]),
    "kv_batch_reserve": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32, _PI32, _PI32]),
    "kv_append": (ctypes.c_int, [_P, _I32, _P, _P, _P, _I32, _P]),
    "paged_attention_workspace_bytes": (_I64, [_P, _I32, _I32, _I32, _I32]),
    "paged_attention_workspace_init": (ctypes.c_int, [_P, _P, _I64, _P]),
    "paged_attention_decode": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                              _I32, ctypes.c_float, _I32, _P, _I64, _P]),
    "paged_attention_decode_append": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _P, _P, _P, _I32,
                                                     _P, _I32, _I32, _I32, ctypes.c_float, _I32, _P,
                                                     _I64, _P]),
    "paged_attention_decode_append_noalloc": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _P, _P, _P, _I32,
                                                             _P, _I32, _I32, _I32, ctypes.c_float, _I32, _P]),
    "kv_prefix_match": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32, _I32, _PI32]),
    "kv_prefix_insert": (ctypes.c_int, [_P, _I64, _PI32, _I32, _PI32, _I32, _PI32]),
    "kv_prefix_evict": (ctypes.c_int, [_P, _I32, _PI32, _PI32]),
    "kv_prefix_num_entries": (ctypes.c_int, [_P, _PI32]),
    "kv_batch_reserve_cow": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32, _PI32, _PI32, _PI32, _PI32,
                                            _PI32]),
    "kv_block_copy": (ctypes.c_int, [_P, _P, _P, _I32, _P]),
    "paged_attention_decode_window": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _I32, _I32,
                                                     _I32, ctypes.c_float, _I32, _I32, _I32, _P, _I64,
                                                     _P]),
    "paged_attention_decode_window_append": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _P, _P, _P, _I32,
                                                            _P, _I32, _I32, _I32, ctypes.c_float, _I32, _I32,
                                                            _I32, _P, _I64, _P]),
    "kv_window_release": (ctypes.c_int, [_P, _I32, _PI32, _I32, _PI32, _I32, _I32, _PI32]),
    "paged_attention_prefill": (ctypes.c_int, [_P, _I32, _P, _P, _I32, _P, _I32, _P, _P, _I32, _I32, _I32,
                                               _I32, ctypes.c_float, _P]),
    # pagedkv_probe.h (a measurement aid, not part of the attention path)
    "kv_probe_gather": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _P, _I32, _P]),
    "kv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kv_last_error": (ctypes.c_char_p, []),
}

_lib = None


class KVError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


def load_library(path=None):
    """Load libpagedkv.so (built in-tree by paged_kv_cache_271_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("PAGEDKV_LIB") or LIB_PATH
    if not path.endswith("_host_san.so"):
        # torch first: it brings its own HIP runtime, and the library must bind
        # to that same runtime (loaded first, the library would pull in the
        # system one, and the two do not share devices or memory).  The
        # host-only sanitizer build has no device code and no HIP runtime.
        import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(f"libpagedkv.so not built at {path}; run "
                          "`python -m paged_kv_cache_271_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        raise KVError(status, _lib.kv_last_error().decode())


def _i32p(a):
    return a.ctypes.data_as(_PI32)


def _host_i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def _dev_ptr(t, what, dtype=None, numel=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a torch tensor on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ sizes ----
def make_desc(num_layers, num_blocks, num_kv_heads, head_dim, cache_dtype, block_size=BLOCK_SIZE):
    if isinstance(cache_dtype, str):
        cache_dtype = DTYPE_NAMES[cache_dtype]
    return KvPoolDesc(num_layers, num_blocks, block_size, num_kv_heads, head_dim, cache_dtype)


def kv_bytes_per_token(desc):
    load_library()
    return _lib.kv_bytes_per_token(ctypes.byref(desc))


def kv_blocks_for_tokens(n, block_size=BLOCK_SIZE):
    load_library()
    return _lib.kv_blocks_for_tokens(n, block_size)


def kv_pool_buffer_bytes(desc):
    load_library()
    cb, sb = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.kv_pool_buffer_bytes(ctypes.byref(desc), ctypes.byref(cb), ctypes.byref(sb)))
    return cb.value, sb.value


# ------------------------------------------------------------------- pool ----
def kv_pool_create(desc, k_cache, v_cache, k_scale=None, v_scale=None, initial_free_order=None):
    """Returns an opaque handle (ctypes.c_void_p).  Buffers are device tensors."""
    load_library()
    cb, sb = kv_pool_buffer_bytes(desc)
    kp = _dev_ptr(k_cache, "k_cache")
    vp = _dev_ptr(v_cache, "v_cache")
    for t, what in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.numel() * t.element_size() != cb:
            raise ValueError(f"{what} holds {t.numel() * t.element_size()} bytes, pool needs {cb}")
    ks = vs = None
    if k_scale is not None or v_scale is not None:
        import torch
        ks = _dev_ptr(k_scale, "k_scale", torch.float32, sb // 4)
        vs = _dev_ptr(v_scale, "v_scale", torch.float32, sb // 4)
    order = None
    if initial_free_order is not None:
        order_arr = _host_i32(initial_free_order)
        if order_arr.size != desc.num_blocks:
            raise ValueError("initial_free_order must hold num_blocks ids")
        order = _i32p(order_arr)
    h = ctypes.c_void_p()
    _check(_lib.kv_pool_create(ctypes.byref(desc), kp, vp, ks, vs, order, ctypes.byref(h)))
    return h


def kv_pool_destroy(h):
    load_library()
    _check(_lib.kv_pool_destroy(h))


def kv_block_alloc(h):
    b = ctypes.c_int32()
    _check(_lib.kv_block_alloc(h, ctypes.byref(b)))
    return b.value


def kv_block_retain(h, block):
    _check(_lib.kv_block_retain(h, int(block)))


def kv_block_release(h, block):
    _check(_lib.kv_block_release(h, int(block)))


def kv_block_retain_n(h, blocks):
    a = _host_i32(blocks)
    _check(_lib.kv_block_retain_n(h, _i32p(a), a.size))


def kv_block_release_n(h, blocks):
    a = _host_i32(blocks)
    _check(_lib.kv_block_release_n(h, _i32p(a), a.size))


def kv_block_refcount(h, block):
    rc = ctypes.c_int32()
    _check(_lib.kv_block_refcount(h, int(block), ctypes.byref(rc)))
    return rc.value


def kv_num_free_blocks(h):
    n = ctypes.c_int32()
    _check(_lib.kv_num_free_blocks(h, ctypes.byref(n)))
    return n.value


def kv_num_shared_blocks(h):
    n = ctypes.c_int32()
    _check(_lib.kv_num_shared_blocks(h, ctypes.byref(n)))
    return n.value


def kv_slot_mapping(h, table_row, positions):
    t = _host_i32(table_row)
    p = _host_i32(positions)
    out = np.empty(p.size, dtype=np.int32)
    _check(_lib.kv_slot_mapping(h, _i32p(t), t.size, _i32p(p), p.size, _i32p(out)))
    return out


def kv_batch_reserve(h, table, lens, n_new):
    """table: int32 [B, max_blocks] and lens: int32 [B] numpy arrays, updated in
    place; n_new: [B].  Returns the int32 slots of the new positions."""
    if table.dtype != np.int32 or not table.flags.c_contiguous or table.ndim != 2:
        raise TypeError("table must be a C-contiguous int32 [B, max_blocks] array")
    if lens.dtype != np.int32 or not lens.flags.c_contiguous or lens.size != table.shape[0]:
        raise TypeError("lens must be a contiguous int32 [B] array")
    nn = _host_i32(n_new)
    if nn.size != lens.size:
        raise ValueError("n_new must have B entries")
    out = np.empty(int(nn.sum()), dtype=np.int32)
    _check(_lib.kv_batch_reserve(h, lens.size, _i32p(table), table.shape[1], _i32p(lens),
                                 _i32p(nn), _i32p(out)))
    return out


def kv_prefix_match(h, tenant, tokens, max_blocks=None):
    """Pages of the longest cached whole-page prefix of `tokens` (each retained)."""
    t = _host_i32(tokens)
    cap = t.size // 16 if max_blocks is None else int(max_blocks)
    out = np.empty(max(cap, 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(_lib.kv_prefix_match(h, int(tenant), _i32p(t), t.size, _i32p(out), cap, ctypes.byref(n)))
    return out[:n.value].copy()


def kv_prefix_insert(h, tenant, tokens, table_row):
    t = _host_i32(tokens)
    r = _host_i32(table_row)
    n = ctypes.c_int32()
    _check(_lib.kv_prefix_insert(h, int(tenant), _i32p(t), t.size, _i32p(r), r.size, ctypes.byref(n)))
    return n.value


def kv_prefix_evict(h, n_wanted):
    out = np.empty(max(int(n_wanted), 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(_lib.kv_prefix_evict(h, int(n_wanted), _i32p(out), ctypes.byref(n)))
    return out[:n.value].copy()


def kv_prefix_num_entries(h):
    n = ctypes.c_int32()
    _check(_lib.kv_prefix_num_entries(h, ctypes.byref(n)))
    return n.value


def kv_batch_reserve_cow(h, table, lens, n_new):
    """kv_batch_reserve with copy-on-write; returns (slots, copy_src, copy_dst)."""
    if table.dtype != np.int32 or not table.flags.c_contiguous or table.ndim != 2:
        raise TypeError("table must be a C-contiguous int32 [B, max_blocks] array")
    if lens.dtype != np.int32 or not lens.flags.c_contiguous or lens.size != table.shape[0]:
        raise TypeError("lens must be a contiguous int32 [B] array")
    nn = _host_i32(n_new)
    if nn.size != lens.size:
        raise ValueError("n_new must have B entries")
    out = np.empty(int(nn.sum()), dtype=np.int32)
    src = np.empty(max(lens.size, 1), dtype=np.int32)
    dst = np.empty(max(lens.size, 1), dtype=np.int32)
    nc = ctypes.c_int32()
    _check(_lib.kv_batch_reserve_cow(h, lens.size, _i32p(table), table.shape[1], _i32p(lens),
                                     _i32p(nn), _i32p(out), _i32p(src), _i32p(dst), ctypes.byref(nc)))
    return out, src[:nc.value].copy(), dst[:nc.value].copy()


# ------------------------------------------------------------ device ops ----
def kv_block_copy(h, src, dst, stream=None):
    """src, dst: int32 device tensors of page ids (same length)."""
    import torch
    n = src.numel()
    sp = _dev_ptr(src, "src", torch.int32)
    dp = _dev_ptr(dst, "dst", torch.int32, n)
    _check(_lib.kv_block_copy(h, sp, dp, n, _stream_ptr(stream)))


def kv_probe_gather(k_base, v_base, k_offsets, v_offsets, run_bytes, sink, stream=None):
    """Measurement aid: read run_bytes at k_base + k_offsets[i] and v_base +
    v_offsets[i] for every i (int64 device tensors); k_base, v_base: device
    addresses (ints); sink: uint32-sized int32 device tensor, one entry per
    workgroup, receiving XORs of the words read."""
    import torch
    n = k_offsets.numel()
    kp = _dev_ptr(k_offsets, "k_offsets", torch.int64)
    vp = _dev_ptr(v_offsets, "v_offsets", torch.int64, n)
    sp = _dev_ptr(sink, "sink", torch.int32)
    _check(_lib.kv_probe_gather(ctypes.c_void_p(k_base), ctypes.c_void_p(v_base), kp, vp, n, int(run_bytes),
                                sp, sink.numel(), _stream_ptr(stream)))


def kv_append(h, desc, layer, k_new, v_new, slot_mapping, stream=None):
    """k_new, v_new: [T, h_kv, d_h] (float32 for f32 pools, bfloat16 otherwise);
    slot_mapping: int32 [T] on the device."""
    import torch
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    T = slot_mapping.numel()
    n = T * desc.num_kv_heads * desc.head_dim
    kp = _dev_ptr(k_new, "k_new", want, n)
    vp = _dev_ptr(v_new, "v_new", want, n)
    sp = _dev_ptr(slot_mapping, "slot_mapping", torch.int32)
    _check(_lib.kv_append(h, int(layer), kp, vp, sp, T, _stream_ptr(stream)))


def paged_attention_workspace_bytes(h, B, h_q, max_ctx, partition_tokens=0):
    return _lib.paged_attention_workspace_bytes(h, B, h_q, max_ctx, partition_tokens)


def paged_attention_workspace_init(h, workspace, stream=None):
    """Zero the counter region of a decode workspace (uint8 device tensor)."""
    wp = _dev_ptr(workspace, "workspace")
    _check(_lib.paged_attention_workspace_init(h, wp, workspace.numel() * workspace.element_size(),
                                               _stream_ptr(stream)))


def new_workspace(h, nbytes, device, stream=None):
    """A decode workspace of nbytes, allocated for `stream` (the caching
    allocator then reuses it only after that stream's work) with its counter
    region zeroed on that stream; None when nbytes is 0."""
    import torch
    if nbytes <= 0:
        return None
    s = torch.cuda.current_stream(device) if stream is None else stream
    with torch.cuda.stream(s):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    paged_attention_workspace_init(h, ws, s)
    return ws


def paged_attention_decode(h, desc, layer, out, q, block_tables, context_lens, max_ctx, scale,
                           partition_tokens=0, workspace=None, stream=None):
    """q, out: [B, h_q, d_h] (float32 with f32 pools, bfloat16 otherwise);
    block_tables: int32 [B, max_blocks]; context_lens: int32 [B]."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B, h_q, head_dim]")
    B, h_q, _ = q.shape
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    qp = _dev_ptr(q, "q", want)
    op = _dev_ptr(out, "out", want, q.numel())
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    wp, wb = None, 0
    if workspace is not None:
        wp = _dev_ptr(workspace, "workspace")
        wb = workspace.numel() * workspace.element_size()
    qd = KV_F32 if want == torch.float32 else KV_BF16
    _check(_lib.paged_attention_decode(h, int(layer), op, qp, qd, tp, block_tables.shape[1], cp, B,
                                       h_q, int(max_ctx), float(scale), int(partition_tokens), wp,
                                       wb, _stream_ptr(stream)))


def paged_attention_decode_append(h, desc, layer, out, q, k_new, v_new, slot_mapping,
                                  block_tables, context_lens, max_ctx, scale, partition_tokens=0,
                                  workspace=None, stream=None):
    """paged_attention_decode with the step's append: k_new, v_new [B, h_kv, d_h]
    (the pool's input dtype), slot_mapping int32 [B] (-1: no new token)."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B, h_q, head_dim]")
    B, h_q, _ = q.shape
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    qp = _dev_ptr(q, "q", want)
    op = _dev_ptr(out, "out", want, q.numel())
    n = B * desc.num_kv_heads * desc.head_dim
    kp = _dev_ptr(k_new, "k_new", want, n)
    vp = _dev_ptr(v_new, "v_new", want, n)
    sp = _dev_ptr(slot_mapping, "slot_mapping", torch.int32, B)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    wp, wb = None, 0
    if workspace is not None:
        wp = _dev_ptr(workspace, "workspace")
        wb = workspace.numel() * workspace.element_size()
    qd = KV_F32 if want == torch.float32 else KV_BF16
    _check(_lib.paged_attention_decode_append(h, int(layer), op, qp, qd, kp, vp, sp, tp,
                                              block_tables.shape[1], cp, B, h_q, int(max_ctx),
                                              float(scale), int(partition_tokens), wp, wb,
                                              _stream_ptr(stream)))


def paged_attention_decode_append_noalloc(h, desc, layer, out, q, k_new, v_new, slot_mapping, block_tables,
                                          context_lens, max_ctx, scale, partition_tokens=0, stream=None):
    """paged_attention_decode_append with the library's fixed scratch as its
    workspace (no device memory allocated by anyone)."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B, h_q, head_dim]")
    B, h_q, _ = q.shape
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    qp = _dev_ptr(q, "q", want)
    op = _dev_ptr(out, "out", want, q.numel())
    n = B * desc.num_kv_heads * desc.head_dim
    kp = _dev_ptr(k_new, "k_new", want, n)
    vp = _dev_ptr(v_new, "v_new", want, n)
    sp = _dev_ptr(slot_mapping, "slot_mapping", torch.int32, B)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    qd = KV_F32 if want == torch.float32 else KV_BF16
    _check(_lib.paged_attention_decode_append_noalloc(h, int(layer), op, qp, qd, kp, vp, sp, tp,
                                                      block_tables.shape[1], cp, B, h_q, int(max_ctx),
                                                      float(scale), int(partition_tokens), _stream_ptr(stream)))


def paged_attention_decode_window(h, desc, layer, out, q, block_tables, context_lens, max_ctx, scale,
                                  sink_tokens, window_tokens, partition_tokens=0, workspace=None,
                                  stream=None):
    """paged_attention_decode over positions < sink_tokens and the last window_tokens."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B, h_q, head_dim]")
    B, h_q, _ = q.shape
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    qp = _dev_ptr(q, "q", want)
    op = _dev_ptr(out, "out", want, q.numel())
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    wp, wb = None, 0
    if workspace is not None:
        wp = _dev_ptr(workspace, "workspace")
        wb = workspace.numel() * workspace.element_size()
    qd = KV_F32 if want == torch.float32 else KV_BF16
    _check(_lib.paged_attention_decode_window(h, int(layer), op, qp, qd, tp, block_tables.shape[1], cp, B,
                                              h_q, int(max_ctx), float(scale), int(sink_tokens),
                                              int(window_tokens), int(partition_tokens), wp, wb,
                                              _stream_ptr(stream)))


def paged_attention_decode_window_append(h, desc, layer, out, q, k_new, v_new, slot_mapping, block_tables,
                                         context_lens, max_ctx, scale, sink_tokens, window_tokens,
                                         partition_tokens=0, workspace=None, stream=None):
    """paged_attention_decode_window with the step's append (arguments as for
    paged_attention_decode_append)."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [B, h_q, head_dim]")
    B, h_q, _ = q.shape
    want = torch.float32 if desc.cache_dtype == KV_F32 else torch.bfloat16
    qp = _dev_ptr(q, "q", want)
    op = _dev_ptr(out, "out", want, q.numel())
    n = B * desc.num_kv_heads * desc.head_dim
    kp = _dev_ptr(k_new, "k_new", want, n)
    vp = _dev_ptr(v_new, "v_new", want, n)
    sp = _dev_ptr(slot_mapping, "slot_mapping", torch.int32, B)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, max_blocks]")
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    wp, wb = None, 0
    if workspace is not None:
        wp = _dev_ptr(workspace, "workspace")
        wb = workspace.numel() * workspace.element_size()
    qd = KV_F32 if want == torch.float32 else KV_BF16
    _check(_lib.paged_attention_decode_window_append(h, int(layer), op, qp, qd, kp, vp, sp, tp,
                                                     block_tables.shape[1], cp, B, h_q, int(max_ctx),
                                                     float(scale), int(sink_tokens), int(window_tokens),
                                                     int(partition_tokens), wp, wb, _stream_ptr(stream)))


def paged_attention_prefill(h, desc, layer, out, q, block_tables, context_lens, query_start, max_q_len,
                            max_ctx, scale, stream=None):
    """q, out: bf16 [rows, h_q, d_h]; query_start: int32 [B+1] on the device."""
    import torch
    if q.dim() != 3 or q.shape[2] != desc.head_dim:
        raise ValueError("q must be [rows, h_q, head_dim]")
    rows, h_q, _ = q.shape
    qp = _dev_ptr(q, "q", torch.bfloat16)
    op = _dev_ptr(out, "out", torch.bfloat16, q.numel())
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [B, max_blocks]")
    B = block_tables.shape[0]
    tp = _dev_ptr(block_tables, "block_tables", torch.int32)
    cp = _dev_ptr(context_lens, "context_lens", torch.int32, B)
    sp = _dev_ptr(query_start, "query_start", torch.int32, B + 1)
    _check(_lib.paged_attention_prefill(h, int(layer), op, qp, KV_BF16, tp, block_tables.shape[1], cp, sp, B,
                                        h_q, int(max_q_len), int(max_ctx), float(scale), _stream_ptr(stream)))


def kv_window_release(h, table, lens, sink_tokens, window_tokens):
    """Drop the dead pages of every request (table edited in place, -1 marks
    them); returns how many."""
    if table.dtype != np.int32 or not table.flags.c_contiguous or table.ndim != 2:
        raise TypeError("table must be a C-contiguous int32 [B, max_blocks] array")
    ln = _host_i32(lens)
    if ln.size != table.shape[0]:
        raise ValueError("lens must have B entries")
    n = ctypes.c_int32()
    _check(_lib.kv_window_release(h, ln.size, _i32p(table), table.shape[1], _i32p(ln), int(sink_tokens),
                                  int(window_tokens), ctypes.byref(n)))
    return n.value


def kv_status_string(status):
    load_library()
    return _lib.kv_status_string(status).decode()


def kv_last_error():
    load_library()
    return _lib.kv_last_error().decode()


# --------------------------------------------------------- convenience ------
class Pool:
    """A pool over device arrays allocated with torch, plus its handle.

    Attributes k_cache / v_cache ([L, N, h_kv, 16, d] and [L, N, h_kv, d, 16])
    and, for fp8, k_scale / v_scale ([L, N, h_kv] float32) are torch tensors.
    """

    def __init__(self, num_layers, num_blocks, num_kv_heads, head_dim, dtype="bf16",
                 device="cuda", initial_free_order=None):
        import torch
        load_library()
        self.desc = make_desc(num_layers, num_blocks, num_kv_heads, head_dim, dtype)
        self.dtype = dtype
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "int8": torch.int8}[dtype]
        L, N, H, D, bs = num_layers, num_blocks, num_kv_heads, head_dim, BLOCK_SIZE
        self.k_cache = torch.zeros((L, N, H, bs, D), dtype=tdt, device=device)
        self.v_cache = torch.zeros((L, N, H, D, bs), dtype=tdt, device=device)
        self.k_scale = self.v_scale = None
        if dtype in ("fp8", "int8"):
            self.k_scale = torch.zeros((L, N, H), dtype=torch.float32, device=device)
            self.v_scale = torch.zeros((L, N, H), dtype=torch.float32, device=device)
        self.handle = kv_pool_create(self.desc, self.k_cache, self.v_cache, self.k_scale,
                                     self.v_scale, initial_free_order)

    def close(self):
        if getattr(self, "handle", None) is not None:
            kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self):
        return kv_block_alloc(self.handle)

    def retain(self, b):
        kv_block_retain(self.handle, b)

    def release(self, b):
        kv_block_release(self.handle, b)

    def retain_n(self, blocks):
        kv_block_retain_n(self.handle, blocks)

    def release_n(self, blocks):
        kv_block_release_n(self.handle, blocks)

    def refcount(self, b):
        return kv_block_refcount(self.handle, b)

    def num_free(self):
        return kv_num_free_blocks(self.handle)

    def num_shared(self):
        return kv_num_shared_blocks(self.handle)

    def slot_mapping(self, table_row, positions):
        return kv_slot_mapping(self.handle, table_row, positions)

    def batch_reserve(self, table, lens, n_new):
        return kv_batch_reserve(self.handle, table, lens, n_new)

    def prefix_match(self, tenant, tokens, max_blocks=None):
        return kv_prefix_match(self.handle, tenant, tokens, max_blocks)

    def prefix_insert(self, tenant, tokens, table_row):
        return kv_prefix_insert(self.handle, tenant, tokens, table_row)

    def prefix_evict(self, n_wanted):
        return kv_prefix_evict(self.handle, n_wanted)

    def prefix_num_entries(self):
        return kv_prefix_num_entries(self.handle)

    def batch_reserve_cow(self, table, lens, n_new):
        return kv_batch_reserve_cow(self.handle, table, lens, n_new)

    def block_copy(self, src, dst, stream=None):
        kv_block_copy(self.handle, src, dst, stream)

    def append(self, layer, k_new, v_new, slot_mapping, stream=None):
        kv_append(self.handle, self.desc, layer, k_new, v_new, slot_mapping, stream)

    def workspace_bytes(self, B, h_q, max_ctx, partition_tokens=0):
        return paged_attention_workspace_bytes(self.handle, B, h_q, max_ctx, partition_tokens)

    def new_workspace(self, B, h_q, max_ctx, partition_tokens=0, device=None, stream=None):
        """A ready decode workspace for this shape (counters zeroed), or None."""
        nbytes = self.workspace_bytes(B, h_q, max_ctx, partition_tokens)
        return new_workspace(self.handle, nbytes, device or self.k_cache.device, stream)

    def decode(self, layer, q, block_tables, context_lens, max_ctx, scale, partition_tokens=0,
               out=None, workspace=None, stream=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.shape[0], q.shape[1], max_ctx, partition_tokens, q.device,
                                           stream)
        paged_attention_decode(self.handle, self.desc, layer, out, q, block_tables, context_lens,
                               max_ctx, scale, partition_tokens, workspace, stream)
        return out

    def decode_window(self, layer, q, block_tables, context_lens, max_ctx, scale, sink_tokens,
                      window_tokens, partition_tokens=0, out=None, workspace=None, stream=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.shape[0], q.shape[1], max_ctx, partition_tokens, q.device,
                                           stream)
        paged_attention_decode_window(self.handle, self.desc, layer, out, q, block_tables, context_lens,
                                      max_ctx, scale, sink_tokens, window_tokens, partition_tokens,
                                      workspace, stream)
        return out

    def decode_window_append(self, layer, q, k_new, v_new, slot_mapping, block_tables, context_lens, max_ctx,
                             scale, sink_tokens, window_tokens, partition_tokens=0, out=None, workspace=None,
                             stream=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.shape[0], q.shape[1], max_ctx, partition_tokens, q.device,
                                           stream)
        paged_attention_decode_window_append(self.handle, self.desc, layer, out, q, k_new, v_new, slot_mapping,
                                             block_tables, context_lens, max_ctx, scale, sink_tokens,
                                             window_tokens, partition_tokens, workspace, stream)
        return out

    def prefill(self, layer, q, block_tables, context_lens, query_start, max_q_len, max_ctx, scale, out=None,
                stream=None):
        import torch
        if out is None:
            out = torch.empty_like(q)
        paged_attention_prefill(self.handle, self.desc, layer, out, q, block_tables, context_lens, query_start,
                                max_q_len, max_ctx, scale, stream)
        return out

    def window_release(self, table, lens, sink_tokens, window_tokens):
        return kv_window_release(self.handle, table, lens, sink_tokens, window_tokens)

    def decode_append(self, layer, q, k_new, v_new, slot_mapping, block_tables, context_lens,
                      max_ctx, scale, partition_tokens=0, out=None, workspace=None, stream=None):
        """Append one token per request (slot_mapping[b], -1 = none), then decode."""
        import torch
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = self.new_workspace(q.shape[0], q.shape[1], max_ctx, partition_tokens, q.device,
                                           stream)
        paged_attention_decode_append(self.handle, self.desc, layer, out, q, k_new, v_new,
                                      slot_mapping, block_tables, context_lens, max_ctx, scale,
                                      partition_tokens, workspace, stream)
        return out
