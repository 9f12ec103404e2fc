"""ctypes binding of libpa.so: the C ABI of include/pa.h under the same names.

Argument marshalling only -- every step of the hot path runs in the library's
HIP kernels or its C++ allocator.  Device calls take torch tensors (device
memory, owned by the caller) and launch on the current torch stream unless a
stream handle is given.  Any non-OK status raises PAError.
"""

import ctypes
import os

import numpy as np
# torch is imported before the library is loaded.  torch ships its own HIP
# runtime (libamdhip64), whose soname the library's dependency matches, so the
# library then binds to that same runtime.  Loaded the other way round, the
# process would hold two HIP runtimes and the library's one sees no device.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same library to load instead (the
# sanitizer build of build.py --sanitize); by default the in-tree libpa.so.
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python paged_kv_cache_424_amd/build.py` "
        "(there is no fallback implementation)")

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({line.split()[-1] for line in f if "libamdhip64" in line})
    except OSError:                                   # pragma: no cover
        return []


if len(_hip_runtimes()) > 1:
    raise ImportError("more than one HIP runtime is loaded in this process "
                      f"({_hip_runtimes()}); load torch before any other HIP library")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_OUT_OF_BLOCKS = -2
PA_ERR_BAD_BLOCK = -3
PA_ERR_BAD_SEQ = -4
PA_ERR_HIP = -5
PA_ERR_UNSUPPORTED = -6
PA_ERR_NO_MEMORY = -7
PA_ERR_TOO_LARGE = -8

# workspace limit of pa_decode_no_alloc (its fixed per-device array)
PA_DECODE_NO_ALLOC_MAX_WORKSPACE = 128 << 20

PA_F32 = 0
PA_BF16 = 1


class PAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {pa_status_string(status)} ({status})"
        if status == PA_ERR_HIP:
            msg += f" [{pa_last_hip_error_name()} = {pa_last_hip_error()}]"
        super().__init__(msg)


class pa_cache_desc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32)]


def cache_desc(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype):
    """kv_dtype: PA_F32 / PA_BF16, or "f32" / "bf16"."""
    if isinstance(kv_dtype, str):
        kv_dtype = {"f32": PA_F32, "bf16": PA_BF16}[kv_dtype]
    return pa_cache_desc(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype)


class pa_allocator_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("num_blocks", "free_blocks", "cached_blocks",
                                              "used_blocks", "shared_blocks", "live_seqs")] + \
               [(n, ctypes.c_int64) for n in ("logical_tokens", "stored_tokens", "hit_tokens",
                                              "evictions")]


_i32, _i64, _f32, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_P32 = ctypes.POINTER(ctypes.c_int32)
_P64 = ctypes.POINTER(ctypes.c_int64)
_PD = ctypes.POINTER(pa_cache_desc)


def _sig(name, res, *args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_lib_status_string = _sig("pa_status_string", ctypes.c_char_p, ctypes.c_int)
_sig("pa_version", _i32)
_sig("pa_last_hip_error", _i32)
_sig("pa_last_hip_error_name", ctypes.c_char_p)
_sig("pa_cache_pool_bytes", _sz, _PD)
_sig("pa_kv_offset", _i64, _PD, _i32, _i64, _i32, _i32)
_sig("pa_allocator_create", ctypes.c_int, _i32, _i32, _P32, ctypes.POINTER(_vp))
_sig("pa_allocator_destroy", None, _vp)
_sig("pa_allocate_block", ctypes.c_int, _vp, _P32)
_sig("pa_free_block", ctypes.c_int, _vp, _i32)
_sig("pa_num_free", _i32, _vp)
_sig("pa_refcount", _i32, _vp, _i32)
_sig("pa_seq_create", ctypes.c_int, _vp, _P32)
_sig("pa_seq_fork", ctypes.c_int, _vp, _i32, _P32)
_sig("pa_seq_append_slots", ctypes.c_int, _vp, _i32, _i32, _P64, _P64, _P32)
_sig("pa_seq_cow_block", ctypes.c_int, _vp, _i32, _i32, _P64, _P32)
_sig("pa_seq_free", ctypes.c_int, _vp, _i32)
_sig("pa_allocator_enable_prefix_cache", ctypes.c_int, _vp)
_sig("pa_num_cached", _i32, _vp)
_sig("pa_seq_append_tokens", ctypes.c_int, _vp, _i32, _P32, _i32, _P64, _P64, _P32, _P32)
_sig("pa_seq_length", _i32, _vp, _i32)
_sig("pa_seq_block_table", ctypes.c_int, _vp, _i32, _P32, _i32, _P32)
_sig("pa_build_block_tables", ctypes.c_int, _vp, _P32, _i32, _i32, _P32, _P32)
_sig("pa_allocator_get_stats", ctypes.c_int, _vp, ctypes.POINTER(pa_allocator_stats))
_sig("pa_cache_write", ctypes.c_int, _vp, _vp, _PD, _vp, _vp, _vp, _i32, _vp)
_sig("pa_copy_blocks", ctypes.c_int, _vp, _vp, _PD, _P64, _i32, _vp)
_sig("pa_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _i32)
_DEC = [_vp, _i32, _vp, _vp, _vp, _PD, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _vp]
_sig("pa_decode", ctypes.c_int, *_DEC)
_sig("pa_decode_partitions", ctypes.c_int, *_DEC)
_sig("pa_decode_no_alloc", ctypes.c_int, *_DEC[:14], _vp)
_sig("pa_decode_reduce", ctypes.c_int, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp)
_sig("pa_time_next_partitions", ctypes.c_int, _vp, _vp)
_DEC_APPEND = [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _PD, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _i32,
               _vp, _sz, _vp]
_sig("pa_decode_append", ctypes.c_int, *_DEC_APPEND)
_sig("pa_decode_append_partitions", ctypes.c_int, *_DEC_APPEND)
_sig("pa_prefill", ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _PD, _vp, _i32, _vp, _vp, _i32, _i32,
     _i32, _i32, _f32, _vp)
_sig("pa_stream_read", ctypes.c_int, _vp, _sz, _i32, _i32, _i32, _vp, _vp)
_sig("pa_attention_loop_peak", ctypes.c_int, _vp, _sz, _i32, _i32, _vp, _P64, _vp)


def _check(rc, where):
    if rc != PA_OK:
        raise PAError(rc, where)


def _i32p(a):
    return a.ctypes.data_as(_P32)


def _i64p(a):
    return a.ctypes.data_as(_P64)


# ---- library / layout ---------------------------------------------------------------
def pa_status_string(status):
    return _lib_status_string(int(status)).decode()


def pa_version():
    return _lib.pa_version()


def pa_last_hip_error():
    return _lib.pa_last_hip_error()


def pa_last_hip_error_name():
    return _lib.pa_last_hip_error_name().decode()


def pa_cache_pool_bytes(desc):
    return _lib.pa_cache_pool_bytes(ctypes.byref(desc))


def pa_kv_offset(desc, which, slot, head, dim):
    return _lib.pa_kv_offset(ctypes.byref(desc), which, slot, head, dim)


# ---- allocator ------------------------------------------------------------------------
def pa_allocator_create(num_blocks, block_size, initial_free_order=None):
    h = _vp()
    order = None
    if initial_free_order is not None:
        order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
        if order.shape != (num_blocks,):
            raise ValueError("initial_free_order must hold num_blocks entries")
    _check(_lib.pa_allocator_create(num_blocks, block_size,
                                    None if order is None else _i32p(order), ctypes.byref(h)),
           "pa_allocator_create")
    return h


def pa_allocator_destroy(h):
    _lib.pa_allocator_destroy(h)


def pa_allocate_block(h):
    b = _i32()
    _check(_lib.pa_allocate_block(h, ctypes.byref(b)), "pa_allocate_block")
    return b.value


def pa_free_block(h, block):
    _check(_lib.pa_free_block(h, block), "pa_free_block")


def pa_num_free(h):
    n = _lib.pa_num_free(h)
    if n < 0:
        raise PAError(n, "pa_num_free")
    return n


def pa_refcount(h, block):
    n = _lib.pa_refcount(h, block)
    if n < 0:
        raise PAError(n, "pa_refcount")
    return n


def pa_seq_create(h):
    s = _i32()
    _check(_lib.pa_seq_create(h, ctypes.byref(s)), "pa_seq_create")
    return s.value


def pa_seq_fork(h, parent):
    s = _i32()
    _check(_lib.pa_seq_fork(h, parent, ctypes.byref(s)), "pa_seq_fork")
    return s.value


def pa_seq_append_slots(h, seq, n_tokens):
    """Returns (slots int64 [n_tokens], cow_pairs list of (src, dst))."""
    slots = np.empty(max(int(n_tokens), 1), dtype=np.int64)
    pair = np.empty(2, dtype=np.int64)
    ncow = _i32()
    _check(_lib.pa_seq_append_slots(h, seq, n_tokens, _i64p(slots), _i64p(pair), ctypes.byref(ncow)),
           "pa_seq_append_slots")
    cow = [(int(pair[0]), int(pair[1]))] if ncow.value else []
    return slots[:n_tokens], cow


def pa_seq_cow_block(h, seq, logical_index):
    pair = np.empty(2, dtype=np.int64)
    ncow = _i32()
    _check(_lib.pa_seq_cow_block(h, seq, logical_index, _i64p(pair), ctypes.byref(ncow)),
           "pa_seq_cow_block")
    return (int(pair[0]), int(pair[1])) if ncow.value else None


def pa_allocator_enable_prefix_cache(h):
    _check(_lib.pa_allocator_enable_prefix_cache(h), "pa_allocator_enable_prefix_cache")


def pa_num_cached(h):
    n = _lib.pa_num_cached(h)
    if n < 0:
        raise PAError(n, "pa_num_cached")
    return n


def pa_seq_append_tokens(h, seq, token_ids):
    """Returns (slots int64 [n], cow_pairs list of (src, dst), n_cached)."""
    toks = np.ascontiguousarray(token_ids, dtype=np.int32).reshape(-1)
    n = len(toks)
    slots = np.empty(max(n, 1), dtype=np.int64)
    pair = np.empty(2, dtype=np.int64)
    ncow = _i32()
    ncached = _i32()
    _check(_lib.pa_seq_append_tokens(h, seq, _i32p(toks) if n else None, n, _i64p(slots), _i64p(pair),
                                     ctypes.byref(ncow), ctypes.byref(ncached)),
           "pa_seq_append_tokens")
    cow = [(int(pair[0]), int(pair[1]))] if ncow.value else []
    return slots[:n], cow, ncached.value


def pa_allocator_get_stats(h):
    """Occupancy counts of the pool as a dict (fields of pa_allocator_stats)."""
    st = pa_allocator_stats()
    _check(_lib.pa_allocator_get_stats(h, ctypes.byref(st)), "pa_allocator_get_stats")
    return {name: int(getattr(st, name)) for name, _ in pa_allocator_stats._fields_}


def pa_seq_free(h, seq):
    _check(_lib.pa_seq_free(h, seq), "pa_seq_free")


def pa_seq_length(h, seq):
    n = _lib.pa_seq_length(h, seq)
    if n < 0:
        raise PAError(n, "pa_seq_length")
    return n


def pa_seq_block_table(h, seq):
    n = _i32()
    rc = _lib.pa_seq_block_table(h, seq, None, 0, ctypes.byref(n))
    if rc not in (PA_OK, PA_ERR_INVALID_ARG):
        _check(rc, "pa_seq_block_table")
    out = np.empty(max(n.value, 1), dtype=np.int32)
    _check(_lib.pa_seq_block_table(h, seq, _i32p(out), out.size, ctypes.byref(n)), "pa_seq_block_table")
    return out[:n.value]


def pa_build_block_tables(h, seqs, max_blocks):
    seqs = np.ascontiguousarray(seqs, dtype=np.int32)
    tables = np.empty((len(seqs), max(max_blocks, 1)), dtype=np.int32)
    lens = np.empty(max(len(seqs), 1), dtype=np.int32)
    _check(_lib.pa_build_block_tables(h, _i32p(seqs), len(seqs), max_blocks, _i32p(tables), _i32p(lens)),
           "pa_build_block_tables")
    return tables[:, :max_blocks], lens[:len(seqs)]


# ---- device ops -----------------------------------------------------------------------
def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _out_dtype(t):
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError("out must be float32 or bfloat16")


def pa_cache_write(k_cache, v_cache, desc, k_new, v_new, slot_mapping, stream=None):
    _check(_lib.pa_cache_write(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc),
                               _dev(k_new, "k_new"), _dev(v_new, "v_new"),
                               _dev(slot_mapping, "slot_mapping"), int(slot_mapping.numel()),
                               _stream(stream)), "pa_cache_write")


def pa_copy_blocks(k_cache, v_cache, desc, pairs, stream=None):
    """pairs: host sequence of (src, dst)."""
    arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
    _check(_lib.pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), ctypes.byref(desc),
                               _i64p(arr) if len(arr) else None, len(arr), _stream(stream)),
           "pa_copy_blocks")


def pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size=0):
    return _lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                          partition_size)


def _decode_args(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len, scale,
                 partition_size, workspace, stream):
    num_seqs, num_q_heads = int(q.shape[0]), int(q.shape[1])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_dev(out, "out"), _out_dtype(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
            _dev(v_cache, "v_cache"), ctypes.byref(desc), _dev(block_tables, "block_tables"),
            int(block_tables.shape[1]), _dev(context_lens, "context_lens"), num_seqs, num_q_heads,
            int(max_context_len), float(scale), int(partition_size), _dev(workspace, "workspace"),
            ws_bytes, _stream(stream))


def pa_decode(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len, scale,
              partition_size=0, workspace=None, stream=None):
    _check(_lib.pa_decode(*_decode_args(out, q, k_cache, v_cache, desc, block_tables, context_lens,
                                        max_context_len, scale, partition_size, workspace, stream)),
           "pa_decode")


def pa_decode_no_alloc(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len, scale,
                       partition_size=0, stream=None):
    """pa_decode with the library's fixed per-device workspace (no allocation)."""
    d = _decode_args(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len, scale,
                     partition_size, None, stream)
    _check(_lib.pa_decode_no_alloc(*d[:14], d[16]), "pa_decode_no_alloc")


def pa_decode_partitions(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len,
                         scale, partition_size=0, workspace=None, stream=None):
    _check(_lib.pa_decode_partitions(*_decode_args(out, q, k_cache, v_cache, desc, block_tables,
                                                   context_lens, max_context_len, scale,
                                                   partition_size, workspace, stream)),
           "pa_decode_partitions")


def _append_args(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, desc, block_tables,
                 context_lens, max_context_len, scale, partition_size, workspace, stream):
    d = _decode_args(out, q, k_cache, v_cache, desc, block_tables, context_lens, max_context_len,
                     scale, partition_size, workspace, stream)
    return d[:3] + (_dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping")) + d[3:]


def pa_decode_append(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, desc, block_tables,
                     context_lens, max_context_len, scale, partition_size=0, workspace=None, stream=None):
    """pa_cache_write of each sequence's newest token (k_new/v_new [B][Hkv][D] at
    slot_mapping[s], int64 [B]) and pa_decode, in one pass."""
    _check(_lib.pa_decode_append(*_append_args(out, q, k_new, v_new, slot_mapping, k_cache, v_cache,
                                               desc, block_tables, context_lens, max_context_len,
                                               scale, partition_size, workspace, stream)),
           "pa_decode_append")


def pa_decode_append_partitions(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, desc,
                                block_tables, context_lens, max_context_len, scale, partition_size=0,
                                workspace=None, stream=None):
    _check(_lib.pa_decode_append_partitions(*_append_args(out, q, k_new, v_new, slot_mapping, k_cache,
                                                          v_cache, desc, block_tables, context_lens,
                                                          max_context_len, scale, partition_size,
                                                          workspace, stream)),
           "pa_decode_append_partitions")


def pa_time_next_partitions(start, stop):
    """Have the next partition pass (pa_decode_partitions or
    pa_decode_append_partitions) of this thread record start / stop
    (torch.cuda.Event, already recorded once so their HIP events exist) at its
    kernel's own dispatch start and end."""
    def handle(ev):
        if ev is None:
            return None
        h = int(ev.cuda_event)
        if not h:
            raise ValueError("event has no HIP event yet: record it once first")
        return ctypes.c_void_p(h)
    _check(_lib.pa_time_next_partitions(handle(start), handle(stop)), "pa_time_next_partitions")


def pa_decode_reduce(out, context_lens, num_q_heads, head_dim, max_context_len, partition_size=0,
                     workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_reduce(_dev(out, "out"), _out_dtype(out), _dev(context_lens, "context_lens"),
                                 int(context_lens.numel()), num_q_heads, head_dim, int(max_context_len),
                                 int(partition_size), _dev(workspace, "workspace"), ws_bytes,
                                 _stream(stream)), "pa_decode_reduce")


def pa_prefill(out, q, k_cache, v_cache, desc, block_tables, context_lens, query_start_loc,
               max_query_len, scale, stream=None):
    _check(_lib.pa_prefill(_dev(out, "out"), _out_dtype(out), _dev(q, "q"), _dev(k_cache, "k_cache"),
                           _dev(v_cache, "v_cache"), ctypes.byref(desc), _dev(block_tables, "block_tables"),
                           int(block_tables.shape[1]), _dev(context_lens, "context_lens"),
                           _dev(query_start_loc, "query_start_loc"), int(context_lens.numel()),
                           int(q.shape[0]), int(q.shape[1]), int(max_query_len), float(scale),
                           _stream(stream)),
           "pa_prefill")


def pa_stream_read(src, sink, blocks_per_cu=8, unroll=4, blocked=0, stream=None):
    """Plain streaming read of the whole device tensor src (a measurement
    yardstick, not part of the attention path); sink: a device tensor of at
    least 4 bytes."""
    _check(_lib.pa_stream_read(_dev(src, "src"), src.numel() * src.element_size(), int(blocks_per_cu),
                               int(unroll), int(blocked), _dev(sink, "sink"), _stream(stream)),
           "pa_stream_read")


def pa_attention_loop_peak(src, sink, iters, mode=2, stream=None):
    """The prefill inner loop's practical ceiling (see pa_measure.h); returns
    the launch's MFMA flops."""
    flops = ctypes.c_int64(0)
    _check(_lib.pa_attention_loop_peak(_dev(src, "src"), src.numel() * src.element_size(), int(iters), int(mode),
                                       _dev(sink, "sink"), ctypes.byref(flops), _stream(stream)),
           "pa_attention_loop_peak")
    return flops.value
