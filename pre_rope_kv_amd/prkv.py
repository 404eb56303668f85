"""Thin ctypes binding of libprkv.so (C ABI in include/prkv.h), same names.

Argument marshalling only: device buffers are passed as raw pointers taken
from torch tensors (``tensor.data_ptr()``) or plain ints; host arrays as
NumPy int32 arrays; streams as ``torch.cuda.Stream`` objects, raw handles or
None (the current torch stream).  Every step of the path runs in the native
library.  A missing library is an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprkv.so")

PRKV_OK = 0
ERRORS = {
    -1: "INVALID_ARG", -2: "ALIGNMENT", -3: "UNKNOWN_FACT", -4: "DUPLICATE_FACT",
    -5: "CAPACITY", -6: "OUT_OF_RANGE", -7: "DUPLICATE_SLOT", -8: "BUFFER_TOO_SMALL",
    -9: "NO_DEVICE", -10: "HIP", -11: "NO_MEMORY",
}
CODES = {v: k for k, v in ERRORS.items()}

# Names the header declares; the library must export every one of them.
EXPORTS = ["store_required_bytes", "store_create", "store_put_fact", "store_stage_facts",
           "store_fact_info",
           "store_destroy", "build_slot_mapping", "inject_topk", "rope_table_fill",
           "last_error_string", "store_upload_fact_table", "inject_device_workspace_bytes",
           "inject_topk_device", "inject_topk_device_noalloc", "retrieve_workspace_bytes",
           "retrieve_topk", "attend_paged"]

# Size of the library's own workspace for inject_topk_device_noalloc.
NOALLOC_SCRATCH_BYTES = 16 << 20


class PrkvError(RuntimeError):
    def __init__(self, code, func, msg):
        self.code = code
        self.name = ERRORS.get(code, str(code))
        super().__init__(f"{func}: PRKV_ERR_{self.name}: {msg}")


class StoreDesc(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_facts", ctypes.c_int32),
        ("capacity_rows", ctypes.c_int64),
        ("max_position", ctypes.c_int32),
        ("rope_style", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("key_layout", ctypes.c_int32),
        ("rope_scaling", ctypes.c_int32),
        ("scaling_factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
        ("original_max_position", ctypes.c_int32),
        ("cache_layout", ctypes.c_int32),
    ]


class DeviceBatch(ctypes.Structure):
    """prkv_device_batch: device pointers describing a batch of requests."""
    _fields_ = [
        ("n_req", ctypes.c_int32),
        ("bt_stride", ctypes.c_int32),
        ("max_facts", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
        ("req_fact_ptr", ctypes.c_void_p),
        ("fact_ids", ctypes.c_void_p),
        ("start_pos", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("bt_len", ctypes.c_void_p),
    ]


class AttnBatch(ctypes.Structure):
    """prkv_attn_batch: device pointers of a query-prefill attention batch."""
    _fields_ = [
        ("n_req", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("bt_stride", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_start", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("bt_len", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("q_lens", ctypes.c_void_p),
    ]


_lib = None
_vp = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """Load libprkv.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m pre_rope_kv_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "store_required_bytes": (ctypes.c_int, [ctypes.POINTER(StoreDesc),
                                                ctypes.POINTER(ctypes.c_size_t),
                                                ctypes.POINTER(ctypes.c_size_t)]),
        "store_create": (ctypes.c_int, [ctypes.POINTER(StoreDesc), _vp, _vp, _vp, _vp,
                                        ctypes.POINTER(_vp)]),
        "store_put_fact": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
        "store_stage_facts": (ctypes.c_int, [_vp, _vp, ctypes.c_int32, _vp, _vp]),
        "store_fact_info": (ctypes.c_int, [_vp, ctypes.c_int32, _i64p, _i32p]),
        "store_destroy": (None, [_vp]),
        "build_slot_mapping": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, _vp, _vp, _vp,
                                              ctypes.c_int32, _vp, ctypes.c_int32,
                                              ctypes.c_int64, _vp, _vp, _vp, ctypes.c_int64,
                                              _i64p]),
        "inject_topk": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp, _vp,
                                       ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                       ctypes.c_int32, ctypes.c_int64, _vp, _vp]),
        "rope_table_fill": (ctypes.c_int, [ctypes.POINTER(StoreDesc), _vp, ctypes.c_size_t]),
        "store_upload_fact_table": (ctypes.c_int, [_vp, _vp, ctypes.c_size_t, _vp]),
        "inject_device_workspace_bytes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64,
                                                         ctypes.POINTER(ctypes.c_size_t)]),
        "inject_topk_device": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(DeviceBatch),
                                              ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                              ctypes.c_int32, ctypes.c_int64, _vp,
                                              ctypes.c_size_t, _vp, _vp]),
        "inject_topk_device_noalloc": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(DeviceBatch),
                                                      ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                      ctypes.c_int32, ctypes.c_int64, _vp, _vp]),
        "retrieve_workspace_bytes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_size_t)]),
        "retrieve_topk": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         _vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp,
                                         _vp, ctypes.c_size_t, _vp, _vp]),
        "attend_paged": (ctypes.c_int, [_vp, ctypes.POINTER(AttnBatch), ctypes.POINTER(_vp),
                                        ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_float, _vp, _vp]),
        "last_error_string": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(rc, func):
    if rc != PRKV_OK:
        msg = lib().last_error_string().decode(errors="replace")
        raise PrkvError(rc, func, msg)


def _ptr(x):
    """Raw address of a torch tensor / numpy array / int / None."""
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


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


ROPE_HALF_SPLIT, ROPE_INTERLEAVED = 0, 1
SCALING_NONE, SCALING_LLAMA3 = 0, 1
KEYS_PRE_ROPE, KEYS_CHUNK_LOCAL = 0, 1
CACHE_NHD, CACHE_HND = 0, 1


def desc(num_layers, num_kv_heads, head_dim, max_facts, capacity_rows, max_position,
         rope_theta, rope_style=ROPE_HALF_SPLIT, key_layout=KEYS_PRE_ROPE, llama3_scaling=None,
         cache_layout=CACHE_NHD):
    """prkv_store_desc.  llama3_scaling: None or (factor, low_freq_factor,
    high_freq_factor, original_max_position)."""
    d = StoreDesc(num_layers, num_kv_heads, head_dim, max_facts, capacity_rows,
                  max_position, rope_style, float(rope_theta))
    d.key_layout = key_layout
    d.cache_layout = cache_layout
    if llama3_scaling is not None:
        factor, lo, hi, w = llama3_scaling
        d.rope_scaling = SCALING_LLAMA3
        d.scaling_factor, d.low_freq_factor, d.high_freq_factor = float(factor), float(lo), float(hi)
        d.original_max_position = int(w)
    return d


def store_required_bytes(d):
    a, r = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().store_required_bytes(ctypes.byref(d), ctypes.byref(a), ctypes.byref(r)),
           "store_required_bytes")
    return a.value, r.value


class Store:
    """Owns a prkv_store handle (host metadata); device memory stays the caller's."""

    def __init__(self, handle, d, keepalive=()):
        self.handle = handle
        self.desc = d
        self._keep = keepalive

    def close(self):
        if self.handle:
            lib().store_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def store_create(d, k_arena=None, v_arena=None, rope_table=None, stream=None):
    h = _vp()
    dev = k_arena is not None or v_arena is not None or rope_table is not None
    s = _stream(stream) if dev else None
    _check(lib().store_create(ctypes.byref(d), _ptr(k_arena), _ptr(v_arena), _ptr(rope_table),
                              s, ctypes.byref(h)), "store_create")
    return Store(h, d, keepalive=(k_arena, v_arena, rope_table))


def store_put_fact(st, fact_id, length, k_src=None, v_src=None, stream=None):
    s = _stream(stream) if k_src is not None else None
    _check(lib().store_put_fact(st.handle, int(fact_id), int(length), _ptr(k_src), _ptr(v_src),
                                s), "store_put_fact")


def store_stage_facts(src, dst, fact_ids, stream=None):
    """Copy the listed facts' K/V rows from store `src` into store `dst`
    (refreshing facts dst already holds, appending the others)."""
    ids = np.ascontiguousarray(np.asarray(fact_ids, dtype=np.int32))
    _check(lib().store_stage_facts(src.handle, dst.handle, int(ids.size),
                                   ids.ctypes.data if ids.size else None, _stream(stream)),
           "store_stage_facts")


def store_fact_info(st, fact_id):
    row, ln = ctypes.c_int64(), ctypes.c_int32()
    _check(lib().store_fact_info(st.handle, int(fact_id), ctypes.byref(row), ctypes.byref(ln)),
           "store_fact_info")
    return row.value, ln.value


def store_destroy(st):
    st.close()


def build_slot_mapping(st, req_fact_ptr, fact_ids, start_pos, block_tables, bt_len,
                       block_size, num_blocks, out=None):
    """Returns (src_row, pos, slot) int32 host arrays of length n_tokens.

    block_tables: int32 [n_req][bt_stride].  out: optional preallocated
    (src_row, pos, slot) arrays (e.g. pinned) with room for the tokens.
    """
    req_fact_ptr, fact_ids, start_pos, bt_len = (_i32(a) for a in
                                                 (req_fact_ptr, fact_ids, start_pos, bt_len))
    bt = _i32(block_tables)
    n_req = len(req_fact_ptr) - 1
    stride = bt.shape[1] if bt.ndim == 2 else 0
    n = ctypes.c_int64()
    if out is None:
        rc = lib().build_slot_mapping(st.handle, n_req, _ptr(req_fact_ptr), _ptr(fact_ids),
                                      _ptr(start_pos), _ptr(bt), stride, _ptr(bt_len),
                                      int(block_size), int(num_blocks), None, None, None, 0,
                                      ctypes.byref(n))
        if rc != CODES["BUFFER_TOO_SMALL"]:
            _check(rc, "build_slot_mapping")
        cap = n.value
        out = tuple(np.empty(cap, np.int32) for _ in range(3))
    cap = min(len(o) for o in out)
    rc = lib().build_slot_mapping(st.handle, n_req, _ptr(req_fact_ptr), _ptr(fact_ids),
                                  _ptr(start_pos), _ptr(bt), stride, _ptr(bt_len),
                                  int(block_size), int(num_blocks), _ptr(out[0]), _ptr(out[1]),
                                  _ptr(out[2]), cap, ctypes.byref(n))
    _check(rc, "build_slot_mapping")
    return tuple(o[:n.value] for o in out)


def inject_topk(st, n_tokens, d_src_row, d_pos, d_slot, k_cache_layers, v_cache_layers,
                block_size, num_blocks, d_status=None, stream=None):
    L = len(k_cache_layers)
    if len(v_cache_layers) != L or L != st.desc.num_layers:
        raise ValueError("need one K and one V cache pointer per layer")
    kp = (_vp * L)(*[_ptr(t) for t in k_cache_layers])
    vp = (_vp * L)(*[_ptr(t) for t in v_cache_layers])
    _check(lib().inject_topk(st.handle, int(n_tokens), _ptr(d_src_row), _ptr(d_pos),
                             _ptr(d_slot), kp, vp, int(block_size), int(num_blocks),
                             _ptr(d_status), _stream(stream)), "inject_topk")


def rope_table_fill(d):
    _, nbytes = store_required_bytes(d)
    out = np.empty(nbytes // 4, np.float32)
    _check(lib().rope_table_fill(ctypes.byref(d), out.ctypes.data, nbytes), "rope_table_fill")
    return out.reshape(d.max_position, d.head_dim // 2, 4)


def store_upload_fact_table(st, d_table, stream=None):
    """d_table: device int32 tensor with >= 2 * max_facts entries."""
    nbytes = d_table.numel() * d_table.element_size() if hasattr(d_table, "numel") else None
    if nbytes is None:
        raise TypeError("d_table must be a device tensor")
    _check(lib().store_upload_fact_table(st.handle, _ptr(d_table), nbytes, _stream(stream)),
           "store_upload_fact_table")


def inject_device_workspace_bytes(max_facts, max_tokens):
    n = ctypes.c_size_t()
    _check(lib().inject_device_workspace_bytes(int(max_facts), int(max_tokens), ctypes.byref(n)),
           "inject_device_workspace_bytes")
    return n.value


def workspace_layout(max_facts, max_tokens):
    """Byte offsets of the workspace parts, as include/prkv.h documents them."""
    def up(v):
        return (v + 255) // 256 * 256
    plan = 256
    src_row = plan + up(max_facts * 16)
    pos = src_row + up(max_tokens * 4)
    slot = pos + up(max_tokens * 4)
    table = slot + up(max_tokens * 4)
    entries = 64
    while entries < 2 * max_tokens:
        entries *= 2
    return {"n_tokens": 0, "n_facts": 8, "plan": plan, "src_row": src_row, "pos": pos,
            "slot": slot, "slot_table": table, "slot_table_entries": entries,
            "total": table + 4 * entries}


BATCH_CHECK_SLOTS = 1


def device_batch(n_req, bt_stride, max_facts, max_tokens, req_fact_ptr, fact_ids, start_pos,
                 block_tables, bt_len, flags=0):
    """prkv_device_batch over device tensors; it holds raw pointers only, so
    the caller keeps the tensors alive while the batch is in use.  flags:
    0 or BATCH_CHECK_SLOTS (detect duplicate slots on the device)."""
    return DeviceBatch(int(n_req), int(bt_stride), int(max_facts), int(flags), int(max_tokens),
                       _ptr(req_fact_ptr), _ptr(fact_ids), _ptr(start_pos),
                       _ptr(block_tables), _ptr(bt_len))


def inject_topk_device(st, d_fact_table, batch, k_cache_layers, v_cache_layers, block_size,
                       num_blocks, d_workspace, workspace_bytes, d_status=None, stream=None):
    L = len(k_cache_layers)
    if len(v_cache_layers) != L or L != st.desc.num_layers:
        raise ValueError("need one K and one V cache pointer per layer")
    kp = (_vp * L)(*[_ptr(t) for t in k_cache_layers])
    vp = (_vp * L)(*[_ptr(t) for t in v_cache_layers])
    _check(lib().inject_topk_device(st.handle, _ptr(d_fact_table), ctypes.byref(batch), kp, vp,
                                    int(block_size), int(num_blocks), _ptr(d_workspace),
                                    int(workspace_bytes), _ptr(d_status), _stream(stream)),
           "inject_topk_device")


def inject_topk_device_noalloc(st, d_fact_table, batch, k_cache_layers, v_cache_layers,
                               block_size, num_blocks, d_status=None, stream=None):
    """inject_topk_device on the library's own per-GPU workspace (no allocation)."""
    L = len(k_cache_layers)
    if len(v_cache_layers) != L or L != st.desc.num_layers:
        raise ValueError("need one K and one V cache pointer per layer")
    kp = (_vp * L)(*[_ptr(t) for t in k_cache_layers])
    vp = (_vp * L)(*[_ptr(t) for t in v_cache_layers])
    _check(lib().inject_topk_device_noalloc(st.handle, _ptr(d_fact_table), ctypes.byref(batch),
                                            kp, vp, int(block_size), int(num_blocks),
                                            _ptr(d_status), _stream(stream)),
           "inject_topk_device_noalloc")


def retrieve_workspace_bytes(n_req, facts_per_store):
    n = ctypes.c_size_t()
    _check(lib().retrieve_workspace_bytes(int(n_req), int(facts_per_store), ctypes.byref(n)),
           "retrieve_workspace_bytes")
    return n.value


def retrieve_topk(d_fact_emb, n_stores, facts_per_store, dim, d_query_emb, d_req_store, n_req,
                  k, d_fact_ids, d_workspace, workspace_bytes, d_scores=None, d_status=None,
                  stream=None):
    _check(lib().retrieve_topk(_ptr(d_fact_emb), int(n_stores), int(facts_per_store), int(dim),
                               _ptr(d_query_emb), _ptr(d_req_store), int(n_req), int(k),
                               _ptr(d_fact_ids), _ptr(d_scores), _ptr(d_workspace),
                               int(workspace_bytes), _ptr(d_status), _stream(stream)),
           "retrieve_topk")


def attn_batch(n_req, q_len, num_q_heads, bt_stride, q, q_start, block_tables, bt_len, out,
               q_lens=None):
    """prkv_attn_batch over device tensors (raw pointers: keep the tensors alive).
    q_lens: optional device int32 [n_req], each request's own query length."""
    return AttnBatch(int(n_req), int(q_len), int(num_q_heads), int(bt_stride), _ptr(q),
                     _ptr(q_start), _ptr(block_tables), _ptr(bt_len), _ptr(out), _ptr(q_lens))


def attend_paged(st, batch, k_cache_layers, v_cache_layers, block_size, num_blocks,
                 softmax_scale, d_status=None, stream=None):
    L = len(k_cache_layers)
    if len(v_cache_layers) != L or L != st.desc.num_layers:
        raise ValueError("need one K and one V cache pointer per layer")
    kp = (_vp * L)(*[_ptr(t) for t in k_cache_layers])
    vp = (_vp * L)(*[_ptr(t) for t in v_cache_layers])
    _check(lib().attend_paged(st.handle, ctypes.byref(batch), kp, vp, int(block_size),
                              int(num_blocks), float(softmax_scale), _ptr(d_status),
                              _stream(stream)), "attend_paged")
