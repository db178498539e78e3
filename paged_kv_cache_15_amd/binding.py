"""ctypes binding of libpagedkv.so (include/paged_kv.h), argument marshalling only.

Every function here has the name of the C entry point it calls.  Device buffers
may be given as torch tensors (their data pointer is passed) or as raw integer
addresses; streams as torch streams, raw hipStream_t addresses, or None for
torch's current stream.  A non-OK status raises PagedKVError carrying the
library's message.  There is no CPU fallback: if the library is not built, importing
this module fails.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGED_KV_LIBRARY may name another build of the same library (same ABI).
LIB_PATH = os.environ.get("PAGED_KV_LIBRARY") or os.path.join(_HERE, "libpagedkv.so")

PAGED_KV_OK = 0
PAGED_KV_ERR_INVALID_ARG = 1
PAGED_KV_ERR_OUT_OF_BLOCKS = 2
PAGED_KV_ERR_UNSUPPORTED = 3
PAGED_KV_ERR_HIP = 4
PAGED_KV_ERR_NO_SUCH_SEQ = 5
PAGED_KV_ERR_BUFFER_TOO_SMALL = 6

PAGED_KV_F32, PAGED_KV_F16, PAGED_KV_BF16 = 0, 1, 2
PAGED_KV_POOL_HOST_ONLY = 1
PAGED_KV_POOL_PREFIX_CACHE = 2
DTYPE_CODES = {"f32": PAGED_KV_F32, "f16": PAGED_KV_F16, "bf16": PAGED_KV_BF16}


class PagedKVError(RuntimeError):
    def __init__(self, func, status, message):
        super().__init__(f"{func}: {message} (status {status})")
        self.status = status


class paged_kv_pool_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


def make_desc(num_blocks, block_size, num_kv_heads, head_dim, dtype, flags=0):
    if isinstance(dtype, str):
        dtype = DTYPE_CODES[dtype]
    return paged_kv_pool_desc(int(num_blocks), int(block_size), int(num_kv_heads), int(head_dim),
                              int(dtype), int(flags))


_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_descp = ctypes.POINTER(paged_kv_pool_desc)
_i32, _i64, _f32, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGNATURES = {
    "paged_kv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "paged_kv_last_error": (ctypes.c_char_p, []),
    "paged_kv_bytes_per_token": (ctypes.c_uint64, [_i32, _i32, _i32, _i32]),
    "paged_kv_pool_bytes": (_sz, [_descp]),
    "paged_kv_pool_create": (ctypes.c_int, [_descp, _i32p, _vp, _vp, ctypes.POINTER(_vp)]),
    "paged_kv_pool_destroy": (None, [_vp]),
    "paged_kv_pool_buffers": (ctypes.c_int, [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "paged_kv_pool_get_desc": (ctypes.c_int, [_vp, _descp]),
    "paged_kv_seq_create": (ctypes.c_int, [_vp, _i32p]),
    "paged_kv_seq_fork": (ctypes.c_int, [_vp, _i32, _i32p]),
    "paged_kv_seq_append": (ctypes.c_int, [_vp, _i32, _i32, _i32p, _i32p, _i32, _i32p]),
    "paged_kv_append_batch": (ctypes.c_int, [_vp, _i32p, _i32p, _i32, _i32p, _i32p, _i32, _i32p,
                                             _i32p]),
    "paged_kv_seq_free": (ctypes.c_int, [_vp, _i32]),
    "paged_kv_block_tables": (ctypes.c_int, [_vp, _i32p, _i32, _i32, _i32p, _i32p]),
    "paged_kv_seq_info": (ctypes.c_int, [_vp, _i32, _i32p, _i32p]),
    "paged_kv_block_refcount": (ctypes.c_int, [_vp, _i32, _i32p]),
    "paged_kv_stats": (ctypes.c_int, [_vp, _i64p, _i64p, _i64p]),
    "paged_kv_block_hash": (ctypes.c_int, [_vp, _i32p, _i32, _i64, _vp]),
    "paged_kv_seq_create_prefix": (ctypes.c_int, [_vp, _i32p, _i32, _i64, _i32p, _i32p]),
    "paged_kv_seq_append_tokens": (ctypes.c_int, [_vp, _i32, _i32p, _i32, _i32p, _i32p, _i32,
                                                  _i32p]),
    "paged_kv_prefix_stats": (ctypes.c_int, [_vp, _i64p, _i64p, _i64p]),
    "paged_kv_copy_blocks": (ctypes.c_int, [_descp, _vp, _vp, _vp, _i32, _vp]),
    "reshape_and_cache": (ctypes.c_int, [_descp, _vp, _vp, _i64, _i64, _vp, _vp, _vp, _i32, _vp]),
    "paged_attention_auto_partition_tokens": (_i32, [_descp, _i32, _i32, _i32]),
    "paged_attention_workspace_bytes": (_sz, [_descp, _i32, _i32, _i32, _i32]),
    "paged_attention_decode": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp,
                                              _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "paged_attention_partition": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp,
                                                 _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]),
    "paged_attention_decode_static": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp, _i32,
                                                     _vp, _i32, _i32, _i32, _f32, _i32, _vp]),
    "paged_attention_decode_append": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp, _vp,
                                                     _vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32,
                                                     _i32, _vp, _sz, _vp]),
    "paged_attention_reduce": (ctypes.c_int, [_descp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp,
                                              _sz, _vp]),
    "paged_kv_read_bandwidth_probe": (ctypes.c_int, [_vp, _sz, _vp, _vp]),
    "paged_kv_shared_prefix_groups": (ctypes.c_int, [_vp, _i32p, _i32, _i32, _i32, _i32p, _i32p,
                                                     _i32p, _i32p]),
    "paged_attention_shared_prefix_workspace_bytes": (_sz, [_descp, _i32, _i32, _i32, _i32, _i32,
                                                            _i32, _i32]),
    "paged_attention_decode_shared_prefix": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp,
                                                            _i32, _vp, _i32, _i32, _i32, _f32, _vp,
                                                            _vp, _i32, _i32, _i32, _i32, _vp, _sz,
                                                            _vp]),
    "paged_attention_prefill": (ctypes.c_int, [_descp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32,
                                               _vp, _i32, _i32, _i32, _i32, _f32, _vp]),
}


def _load():
    # The library must share torch's HIP runtime (torch's streams and device pointers
    # are only valid there).  torch ships its own libamdhip64 with the same soname;
    # loading torch first makes the dynamic linker bind libpagedkv.so to that copy
    # instead of bringing a second HIP runtime into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (python -m paged_kv_cache_15_amd.build); "
                          "this package has no fallback implementation")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = tuple(_SIGNATURES)


def _check(func, status):
    if status != PAGED_KV_OK:
        msg = lib.paged_kv_last_error().decode() or lib.paged_kv_status_string(status).decode()
        raise PagedKVError(func, status, msg)


def _ptr(x):
    """Device or host address of a torch tensor / numpy array / int / None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _i32_array(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


# ------------------------------------------------------------------ misc ----
def paged_kv_status_string(status):
    return lib.paged_kv_status_string(status).decode()


def paged_kv_last_error():
    return lib.paged_kv_last_error().decode()


def paged_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes):
    return int(lib.paged_kv_bytes_per_token(layers, kv_heads, head_dim, dtype_bytes))


def paged_kv_pool_bytes(desc):
    return int(lib.paged_kv_pool_bytes(ctypes.byref(desc)))


# -------------------------------------------------------- pool + allocator ----
def paged_kv_pool_create(desc, free_order=None, k_pool=None, v_pool=None):
    """Returns an opaque pool handle (int).  free_order: host int sequence or None."""
    handle = _vp()
    if free_order is not None:
        arr, p = _i32_array(free_order)
    else:
        arr, p = None, None
    _check("paged_kv_pool_create",
           lib.paged_kv_pool_create(ctypes.byref(desc), p, _ptr(k_pool), _ptr(v_pool),
                                    ctypes.byref(handle)))
    return handle.value


def paged_kv_pool_destroy(pool):
    lib.paged_kv_pool_destroy(pool)


def paged_kv_pool_buffers(pool):
    k, v = _vp(), _vp()
    _check("paged_kv_pool_buffers", lib.paged_kv_pool_buffers(pool, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def paged_kv_pool_get_desc(pool):
    d = paged_kv_pool_desc()
    _check("paged_kv_pool_get_desc", lib.paged_kv_pool_get_desc(pool, ctypes.byref(d)))
    return d


def paged_kv_seq_create(pool):
    sid = ctypes.c_int32()
    _check("paged_kv_seq_create", lib.paged_kv_seq_create(pool, ctypes.byref(sid)))
    return sid.value


def paged_kv_seq_fork(pool, parent):
    sid = ctypes.c_int32()
    _check("paged_kv_seq_fork", lib.paged_kv_seq_fork(pool, parent, ctypes.byref(sid)))
    return sid.value


def paged_kv_seq_append(pool, seq, n_tokens):
    """Returns (slots int32[n], copies int32[k][2])."""
    slots = np.empty(max(n_tokens, 0), dtype=np.int32)
    copies = np.empty(2, dtype=np.int32)
    nc = ctypes.c_int32()
    _check("paged_kv_seq_append",
           lib.paged_kv_seq_append(pool, seq, n_tokens, slots.ctypes.data_as(_i32p),
                                   copies.ctypes.data_as(_i32p), 1, ctypes.byref(nc)))
    return slots, copies[:2 * nc.value].reshape(-1, 2)


def paged_kv_append_batch(pool, seqs, counts):
    """Returns (slots int32[sum(counts)], copies int32[k][2]).  On failure the
    raised error carries .n_done (sequences appended before the failing one)."""
    s_arr, s_p = _i32_array(seqs)
    c_arr, c_p = _i32_array(counts)
    slots = np.empty(int(c_arr.sum()), dtype=np.int32)
    copies = np.empty(2 * max(1, len(s_arr)), dtype=np.int32)
    nc, nd = ctypes.c_int32(), ctypes.c_int32()
    st = lib.paged_kv_append_batch(pool, s_p, c_p, len(s_arr), slots.ctypes.data_as(_i32p),
                                   copies.ctypes.data_as(_i32p), len(s_arr), ctypes.byref(nc),
                                   ctypes.byref(nd))
    try:
        _check("paged_kv_append_batch", st)
    except PagedKVError as e:
        e.n_done = nd.value
        raise
    return slots, copies[:2 * nc.value].reshape(-1, 2)


def paged_kv_seq_free(pool, seq):
    _check("paged_kv_seq_free", lib.paged_kv_seq_free(pool, seq))


def paged_kv_block_tables(pool, seq_ids, max_blocks=None):
    """Returns (tables int32[n][max_blocks] padded with -1, context_lens int32[n])."""
    ids, ids_p = _i32_array(seq_ids)
    if max_blocks is None:
        max_blocks = max([paged_kv_seq_info(pool, int(s))[1] for s in ids] + [1])
    tables = np.empty((len(ids), max_blocks), dtype=np.int32)
    lens = np.empty(len(ids), dtype=np.int32)
    _check("paged_kv_block_tables",
           lib.paged_kv_block_tables(pool, ids_p, len(ids), max_blocks,
                                     tables.ctypes.data_as(_i32p), lens.ctypes.data_as(_i32p)))
    return tables, lens


def paged_kv_seq_info(pool, seq):
    """Returns (context_len, num_blocks)."""
    L, nb = ctypes.c_int32(), ctypes.c_int32()
    _check("paged_kv_seq_info", lib.paged_kv_seq_info(pool, seq, ctypes.byref(L), ctypes.byref(nb)))
    return L.value, nb.value


def paged_kv_block_refcount(pool, block):
    rc = ctypes.c_int32()
    _check("paged_kv_block_refcount", lib.paged_kv_block_refcount(pool, block, ctypes.byref(rc)))
    return rc.value


def paged_kv_stats(pool):
    """Returns (num_free, num_used, waste_slots)."""
    f, u, w = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("paged_kv_stats", lib.paged_kv_stats(pool, ctypes.byref(f), ctypes.byref(u), ctypes.byref(w)))
    return f.value, u.value, w.value


# -------------------------------------------------------- prefix caching ----
def paged_kv_block_hash(parent, tokens, extra_key=0):
    """Chained block hash: 32 bytes from parent (32 bytes or None) and token ids."""
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    out = ctypes.create_string_buffer(32)
    par = None if parent is None else ctypes.create_string_buffer(bytes(parent), 32)
    _check("paged_kv_block_hash",
           lib.paged_kv_block_hash(par, toks.ctypes.data_as(_i32p), len(toks), int(extra_key), out))
    return out.raw


def paged_kv_seq_create_prefix(pool, prompt, extra_key=0):
    """Returns (seq id, number of prompt tokens taken over from cached blocks)."""
    toks = np.ascontiguousarray(np.asarray(prompt, dtype=np.int32))
    sid, nc = ctypes.c_int32(), ctypes.c_int32()
    _check("paged_kv_seq_create_prefix",
           lib.paged_kv_seq_create_prefix(pool, toks.ctypes.data_as(_i32p), len(toks), int(extra_key),
                                          ctypes.byref(sid), ctypes.byref(nc)))
    return sid.value, nc.value


def paged_kv_seq_append_tokens(pool, seq, tokens):
    """Returns (slots int32[n], copies int32[k][2])."""
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    slots = np.empty(max(len(toks), 1), dtype=np.int32)
    copies = np.empty(2, dtype=np.int32)
    nc = ctypes.c_int32()
    _check("paged_kv_seq_append_tokens",
           lib.paged_kv_seq_append_tokens(pool, seq, toks.ctypes.data_as(_i32p), len(toks),
                                          slots.ctypes.data_as(_i32p), copies.ctypes.data_as(_i32p),
                                          1, ctypes.byref(nc)))
    return slots[:len(toks)], copies[:2 * nc.value].reshape(-1, 2)


def paged_kv_prefix_stats(pool):
    """Returns (cached_blocks, hit_blocks, evictions)."""
    c, h, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check("paged_kv_prefix_stats",
           lib.paged_kv_prefix_stats(pool, ctypes.byref(c), ctypes.byref(h), ctypes.byref(e)))
    return c.value, h.value, e.value


# ------------------------------------------------------------ device ops ----
def paged_kv_copy_blocks(desc, k_pool, v_pool, pairs, n, stream=None):
    _check("paged_kv_copy_blocks",
           lib.paged_kv_copy_blocks(ctypes.byref(desc), _ptr(k_pool), _ptr(v_pool), _ptr(pairs),
                                    int(n), _stream(stream)))


def reshape_and_cache(desc, key, value, k_pool, v_pool, slot_mapping, num_tokens=None,
                      key_stride=None, value_stride=None, stream=None):
    """key/value: [T][Hkv][d] tensors (token stride taken from the tensor unless given)."""
    if num_tokens is None:
        num_tokens = key.shape[0]
    f = "reshape_and_cache"
    for name, t in (("key", key), ("value", value)):
        if _is_tensor(t):
            _expect(f, t.dim() == 3 and tuple(t.shape[1:]) == (desc.num_kv_heads, desc.head_dim)
                    and t.shape[0] >= num_tokens,
                    f"{name} must be [>= {num_tokens}][{desc.num_kv_heads}][{desc.head_dim}] "
                    f"(got {tuple(t.shape)})")
            _expect(f, t.stride(2) == 1 and t.stride(1) == desc.head_dim,
                    f"{name}: heads and dims must be contiguous")
            _expect(f, t.element_size() == _ELEM_BYTES.get(desc.dtype),
                    f"{name} element size does not match the pool")
    if _is_tensor(slot_mapping):
        _check_tensor(f, "slot_mapping", slot_mapping, int32=True)
        _expect(f, slot_mapping.numel() >= num_tokens, "slot_mapping shorter than num_tokens")
    if key_stride is None:
        key_stride = key.stride(0)
    if value_stride is None:
        value_stride = value.stride(0)
    _check("reshape_and_cache",
           lib.reshape_and_cache(ctypes.byref(desc), _ptr(key), _ptr(value), int(key_stride),
                                 int(value_stride), _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping),
                                 int(num_tokens), _stream(stream)))


PARTITION_AUTO = -1


def paged_attention_auto_partition_tokens(desc, num_seqs, num_q_heads, max_context_len):
    """The partition_tokens value PARTITION_AUTO resolves to (0 = stream-K), -1 if invalid."""
    return int(lib.paged_attention_auto_partition_tokens(ctypes.byref(desc), num_seqs,
                                                         num_q_heads, max_context_len))


def paged_attention_workspace_bytes(desc, num_seqs, num_q_heads, max_context_len,
                                    partition_tokens=0):
    return int(lib.paged_attention_workspace_bytes(ctypes.byref(desc), num_seqs, num_q_heads,
                                                   max_context_len, partition_tokens))


_ELEM_BYTES = {PAGED_KV_F32: 4, PAGED_KV_F16: 2, PAGED_KV_BF16: 2}


def _is_tensor(x):
    return hasattr(x, "data_ptr") and hasattr(x, "is_contiguous")


def _expect(func, cond, what):
    if not cond:
        raise ValueError(f"{func}: {what}")


def _check_tensor(func, name, t, shape=None, elem_bytes=None, int32=False):
    """Layout checks on a torch tensor argument (raw addresses are passed unchecked):
    contiguous, int32 when asked, the element size of its storage type, and a shape."""
    if not _is_tensor(t):
        return
    import torch
    _expect(func, t.is_contiguous(), f"{name} must be contiguous")
    if int32:
        _expect(func, t.dtype == torch.int32, f"{name} must be int32 (got {t.dtype})")
    if elem_bytes is not None:
        _expect(func, t.element_size() == elem_bytes,
                f"{name} has {t.element_size()}-byte elements, {elem_bytes} expected")
    if shape is not None:
        _expect(func, tuple(t.shape) == tuple(shape),
                f"{name} has shape {tuple(t.shape)}, {tuple(shape)} expected")


def _check_attn(func, desc, out, out_dtype, q, block_tables, context_lens, num_q_heads,
                workspace):
    _check_tensor(func, "context_lens", context_lens, int32=True)
    _check_tensor(func, "block_tables", block_tables, int32=True)
    nseq = int(context_lens.shape[0])
    if _is_tensor(block_tables):
        _expect(func, block_tables.dim() == 2 and block_tables.shape[0] == nseq,
                f"block_tables must be [{nseq}][max_blocks] (got {tuple(block_tables.shape)})")
    rows = (nseq, int(num_q_heads), int(desc.head_dim))
    _check_tensor(func, "q", q, rows, _ELEM_BYTES.get(desc.dtype))
    _check_tensor(func, "out", out, rows, _ELEM_BYTES.get(out_dtype))
    if workspace is not None and _is_tensor(workspace):
        _expect(func, workspace.is_contiguous(), "workspace must be contiguous")


def _attn_args(func, desc, out, out_dtype, q, k_pool, v_pool, block_tables, context_lens,
               num_q_heads, max_context_len, scale, partition_tokens, workspace, stream):
    if isinstance(out_dtype, str):
        out_dtype = DTYPE_CODES[out_dtype]
    _check_attn(func, desc, out, out_dtype, q, block_tables, context_lens, num_q_heads, workspace)
    ws_bytes = 0 if workspace is None else (workspace.numel() * workspace.element_size()
                                            if hasattr(workspace, "numel") else 0)
    return (ctypes.byref(desc), _ptr(out), int(out_dtype), _ptr(q), _ptr(k_pool), _ptr(v_pool),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
            int(context_lens.shape[0]), int(num_q_heads), int(max_context_len), float(scale),
            int(partition_tokens), _ptr(workspace), ws_bytes, _stream(stream))


def paged_attention_decode(desc, out, out_dtype, q, k_pool, v_pool, block_tables, context_lens,
                           num_q_heads, max_context_len, scale, partition_tokens=0,
                           workspace=None, stream=None):
    """block_tables: int32 [B][max_blocks] device tensor; context_lens: int32 [B] device."""
    _check("paged_attention_decode",
           lib.paged_attention_decode(*_attn_args("paged_attention_decode", desc, out, out_dtype,
                                                  q, k_pool, v_pool,
                                                  block_tables, context_lens, num_q_heads,
                                                  max_context_len, scale, partition_tokens,
                                                  workspace, stream)))


def paged_attention_decode_static(desc, out, out_dtype, q, k_pool, v_pool, block_tables,
                                  context_lens, num_q_heads, max_context_len, scale,
                                  partition_tokens=0, stream=None):
    """paged_attention_decode without a workspace: the library's static scratch."""
    args = _attn_args("paged_attention_decode_static", desc, out, out_dtype, q, k_pool, v_pool,
                      block_tables, context_lens, num_q_heads, max_context_len, scale,
                      partition_tokens, None, stream)
    # the same arguments minus (workspace, workspace_bytes)
    _check("paged_attention_decode_static",
           lib.paged_attention_decode_static(*args[:14], args[16]))


def paged_attention_decode_append(desc, out, out_dtype, q, new_k, new_v, slot_mapping, k_pool,
                                  v_pool, block_tables, context_lens, num_q_heads,
                                  max_context_len, scale, partition_tokens=0, workspace=None,
                                  stream=None):
    """One decode step of a layer: the cache write of the new token of every sequence
    (new_k/new_v [B][Hkv][d] in the pool dtype, slot_mapping int32 [B]) and the
    attention over contexts that include it."""
    f = "paged_attention_decode_append"
    args = _attn_args(f, desc, out, out_dtype, q, k_pool, v_pool, block_tables, context_lens,
                      num_q_heads, max_context_len, scale, partition_tokens, workspace, stream)
    n = int(context_lens.shape[0])
    for name, t in (("new_k", new_k), ("new_v", new_v)):
        if _is_tensor(t):
            _check_tensor(f, name, t)
            _expect(f, tuple(t.shape) == (n, desc.num_kv_heads, desc.head_dim),
                    f"{name} must be [{n}][{desc.num_kv_heads}][{desc.head_dim}] (got {tuple(t.shape)})")
            _expect(f, t.element_size() == _ELEM_BYTES.get(desc.dtype),
                    f"{name} element size does not match the pool")
    if _is_tensor(slot_mapping):
        _check_tensor(f, "slot_mapping", slot_mapping, int32=True)
        _expect(f, slot_mapping.numel() >= n, "slot_mapping shorter than the batch")
    # (desc, out, out_dtype, q) + (new_k, new_v, slots) + (k_pool, v_pool, tables, ...)
    _check(f, lib.paged_attention_decode_append(*args[:4], _ptr(new_k), _ptr(new_v),
                                                _ptr(slot_mapping), *args[4:]))


def paged_attention_partition(desc, out, out_dtype, q, k_pool, v_pool, block_tables, context_lens,
                              num_q_heads, max_context_len, scale, partition_tokens=0,
                              workspace=None, stream=None):
    _check("paged_attention_partition",
           lib.paged_attention_partition(*_attn_args("paged_attention_partition", desc, out,
                                                     out_dtype, q, k_pool, v_pool,
                                                     block_tables, context_lens, num_q_heads,
                                                     max_context_len, scale, partition_tokens,
                                                     workspace, stream)))


def paged_attention_prefill(desc, out, out_dtype, q, q_start, k_pool, v_pool, block_tables,
                            context_lens, num_q_heads, max_q_len, max_context_len, scale,
                            stream=None):
    """q_start: int32 [B+1] device (query rows of sequence s: q_start[s] .. q_start[s+1]-1);
    block_tables: int32 [B][max_blocks] device; context_lens: int32 [B] device."""
    if isinstance(out_dtype, str):
        out_dtype = DTYPE_CODES[out_dtype]
    f = "paged_attention_prefill"
    _check_tensor(f, "context_lens", context_lens, int32=True)
    _check_tensor(f, "block_tables", block_tables, int32=True)
    _check_tensor(f, "q_start", q_start, (int(context_lens.shape[0]) + 1,), int32=True)
    if _is_tensor(q):
        _expect(f, q.dim() == 3 and tuple(q.shape[1:]) == (int(num_q_heads), int(desc.head_dim)),
                f"q must be [rows][{num_q_heads}][{desc.head_dim}] (got {tuple(q.shape)})")
        _check_tensor(f, "q", q, elem_bytes=_ELEM_BYTES.get(desc.dtype))
        _check_tensor(f, "out", out, tuple(q.shape), _ELEM_BYTES.get(out_dtype))
    _check("paged_attention_prefill",
           lib.paged_attention_prefill(ctypes.byref(desc), _ptr(out), int(out_dtype), _ptr(q),
                                       _ptr(q_start), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_tables), int(block_tables.shape[1]),
                                       _ptr(context_lens), int(context_lens.shape[0]),
                                       int(num_q_heads), int(max_q_len), int(max_context_len),
                                       float(scale), _stream(stream)))


def paged_attention_reduce(desc, out, out_dtype, context_lens, num_q_heads, max_context_len,
                           partition_tokens=0, workspace=None, stream=None):
    if isinstance(out_dtype, str):
        out_dtype = DTYPE_CODES[out_dtype]
    f = "paged_attention_reduce"
    _check_tensor(f, "context_lens", context_lens, int32=True)
    _check_tensor(f, "out", out, (int(context_lens.shape[0]), int(num_q_heads), int(desc.head_dim)),
                  _ELEM_BYTES.get(out_dtype))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("paged_attention_reduce",
           lib.paged_attention_reduce(ctypes.byref(desc), _ptr(out), int(out_dtype),
                                      _ptr(context_lens), int(context_lens.shape[0]),
                                      int(num_q_heads), int(max_context_len),
                                      int(partition_tokens), _ptr(workspace), ws_bytes,
                                      _stream(stream)))


# --------------------------------------------------- shared-prefix decode ----
def paged_kv_shared_prefix_groups(pool, seq_ids, max_group, min_shared_tokens=16):
    """Returns (group_start int32[g+1], shared_tokens int32[g], max_shared)."""
    ids, ids_p = _i32_array(seq_ids)
    n = len(ids)
    gs = np.zeros(n + 1, dtype=np.int32)
    sh = np.zeros(max(n, 1), dtype=np.int32)
    ng, ms = ctypes.c_int32(), ctypes.c_int32()
    _check("paged_kv_shared_prefix_groups",
           lib.paged_kv_shared_prefix_groups(pool, ids_p, n, int(max_group), int(min_shared_tokens),
                                             gs.ctypes.data_as(_i32p), sh.ctypes.data_as(_i32p),
                                             ctypes.byref(ng), ctypes.byref(ms)))
    return gs[:ng.value + 1].copy(), sh[:ng.value].copy(), ms.value


def paged_attention_shared_prefix_workspace_bytes(desc, num_seqs, num_q_heads, max_context_len,
                                                  num_groups, max_group, max_shared_tokens,
                                                  partition_tokens=0):
    return int(lib.paged_attention_shared_prefix_workspace_bytes(
        ctypes.byref(desc), int(num_seqs), int(num_q_heads), int(max_context_len),
        int(num_groups), int(max_group), int(max_shared_tokens), int(partition_tokens)))


def paged_attention_decode_shared_prefix(desc, out, out_dtype, q, k_pool, v_pool, block_tables,
                                         context_lens, num_q_heads, max_context_len, scale,
                                         group_start, shared_tokens, num_groups, max_group,
                                         max_shared_tokens, partition_tokens=0, workspace=None,
                                         stream=None):
    """group_start int32 [G+1] and shared_tokens int32 [G]: device tensors."""
    f = "paged_attention_decode_shared_prefix"
    args = _attn_args(f, desc, out, out_dtype, q, k_pool, v_pool, block_tables, context_lens,
                      num_q_heads, max_context_len, scale, partition_tokens, workspace, stream)
    _check_tensor(f, "group_start", group_start, (int(num_groups) + 1,), int32=True)
    _check_tensor(f, "shared_tokens", shared_tokens, (int(num_groups),), int32=True)
    _check(f, lib.paged_attention_decode_shared_prefix(
        *args[:13], _ptr(group_start), _ptr(shared_tokens), int(num_groups), int(max_group),
        int(max_shared_tokens), int(partition_tokens), args[14], args[15], args[16]))


# ------------------------------------------------------------ measurement ----
def paged_kv_read_bandwidth_probe(buf, sink, nbytes=None, stream=None):
    """Streaming read of `buf` (a device tensor, or an address with nbytes given)."""
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check("paged_kv_read_bandwidth_probe",
           lib.paged_kv_read_bandwidth_probe(_ptr(buf), int(nbytes), _ptr(sink), _stream(stream)))
