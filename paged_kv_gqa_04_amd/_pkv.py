"""ctypes binding for ``libpkv.so`` (the C ABI in ``include/pkv.h``).

Argument marshalling only: every step of a decode runs in the library's HIP
kernels. Device buffers may be passed as integers (device addresses) or as
objects with a ``data_ptr()`` method (torch tensors); streams and events as
integer handles. Failing calls raise ``PkvError`` carrying the status code
and the library's message. Importing fails loudly if the library is missing:
there is no fallback implementation.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

# PKV_LIBRARY may name another build of the same ABI (e.g. a tuning variant).
_LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_ERR_STATE = -5
PKV_ERR_POOL = -6

PKV_F16 = 0
PKV_BF16 = 1

PKV_MODE_AUTO = 0
PKV_MODE_UNSPLIT = 1
PKV_MODE_SPLIT = 2
PKV_MODE_WORKQUEUE = 3
PKV_MODE_BUCKETED = 4

MODES = {"auto": PKV_MODE_AUTO, "unsplit": PKV_MODE_UNSPLIT,
         "split": PKV_MODE_SPLIT, "workqueue": PKV_MODE_WORKQUEUE,
         "bucketed": PKV_MODE_BUCKETED}
MODE_NAMES = {v: k for k, v in MODES.items()}
DTYPES = {"f16": PKV_F16, "bf16": PKV_BF16}

PKV_MERGE_FUSED = 0
PKV_MERGE_KERNEL = 1
MERGES = {"fused": PKV_MERGE_FUSED, "kernel": PKV_MERGE_KERNEL}


class pkv_shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("block_table_stride", C.c_int32),
                ("num_pages", C.c_int64), ("dtype", C.c_int32),
                ("sm_scale", C.c_float)]


class pkv_opts(C.Structure):
    _fields_ = [("mode", C.c_int32), ("num_splits", C.c_int32),
                ("chunk_pages", C.c_int32), ("num_cus", C.c_int32),
                ("queue_seed", C.c_uint32), ("merge", C.c_int32),
                ("reserved", C.c_int32 * 2)]


class pkv_plan_stats(C.Structure):
    _fields_ = [("mode", C.c_int32), ("num_splits", C.c_int32),
                ("chunk_pages", C.c_int32), ("grid", C.c_int32),
                ("num_items", C.c_int32), ("empty_items", C.c_int32),
                ("num_slots", C.c_int32), ("launches", C.c_int32),
                ("bucket_launches", C.c_int32), ("reserved", C.c_int32),
                ("kv_tokens", C.c_int64), ("algorithmic_bytes", C.c_int64),
                ("partial_bytes", C.c_int64), ("upload_bytes", C.c_int64),
                ("workspace_bytes", C.c_int64)]


class pkv_workspace_layout(C.Structure):
    _fields_ = [("items_offset", C.c_int64), ("meta_offset", C.c_int64),
                ("counters_offset", C.c_int64), ("m_offset", C.c_int64), ("l_offset", C.c_int64),
                ("acc_offset", C.c_int64), ("total_bytes", C.c_int64),
                ("num_items", C.c_int32), ("num_slots", C.c_int32),
                ("group", C.c_int32), ("num_splits", C.c_int32)]


# Bytes between two rows' merge counters (PKV_COUNTER_STRIDE in pkv.h).
COUNTER_STRIDE = 128

# Every function pkv.h declares, with its C signature.
_P = C.c_void_p
SIGNATURES = {
    "pkv_plan_create": (C.c_int32, [C.POINTER(pkv_shape), C.POINTER(C.c_int32),
                                    C.POINTER(pkv_opts), C.POINTER(_P)]),
    "pkv_plan_update": (C.c_int32, [_P, C.POINTER(C.c_int32)]),
    "pkv_plan_upload_needed": (C.c_int32, [_P, C.POINTER(C.c_int32)]),
    "pkv_plan_workspace_bytes": (C.c_size_t, [_P]),
    "pkv_plan_upload": (C.c_int32, [_P, _P, C.c_size_t, _P]),
    "pkv_plan_stats_get": (C.c_int32, [_P, C.POINTER(pkv_plan_stats)]),
    "pkv_plan_layout_get": (C.c_int32, [_P, C.POINTER(pkv_workspace_layout)]),
    "pkv_plan_queue_get": (C.c_int32, [_P, _P, C.c_size_t]),
    "pkv_decode": (C.c_int32, [_P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_decode_marked": (C.c_int32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_plan_destroy": (None, [_P]),
    "pkv_status_string": (C.c_char_p, [C.c_int32]),
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (C.c_int32, []),
    "pkv_pool_create": (C.c_int32, [C.c_int32, C.POINTER(_P)]),
    "pkv_pool_destroy": (None, [_P]),
    "pkv_pool_free_pages": (C.c_int32, [_P]),
    "pkv_pool_alloc": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32)]),
    "pkv_pool_free": (C.c_int32, [_P, C.POINTER(C.c_int32), C.c_int32]),
    "pkv_append_prepare": (C.c_int32, [_P, C.c_int32, C.c_int32, C.c_int32,
                                       C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                       C.POINTER(C.c_int32)]),
    "pkv_pool_release_row": (C.c_int32, [_P, C.POINTER(C.c_int32), C.c_int32, C.c_int32]),
    "pkv_append": (C.c_int32, [C.POINTER(pkv_shape), _P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_decode_append": (C.c_int32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pkv_stream_read": (C.c_int32, [_P, _P, C.c_int64, C.c_int32, _P, _P]),
    "pkv_paged_read": (C.c_int32, [_P, _P, _P, _P, _P, _P, _P]),
    "pkv_decode_static": (C.c_int32, [_P, _P, _P, _P, _P, _P, _P, _P]),
}

# PKV_STATIC_SCRATCH_BYTES in pkv.h: the largest workspace pkv_decode_static takes.
STATIC_SCRATCH_BYTES = 16 << 20


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with "
            "`python paged_kv_gqa_04_amd/build.py` (no fallback exists)")
    lib = C.CDLL(_LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        msg = LIB.pkv_last_error().decode(errors="replace")
        name = LIB.pkv_status_string(status).decode()
        super().__init__(f"{where}: {name}: {msg}")


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        raise PkvError(status, where)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, block_table_stride,
               num_pages, dtype, sm_scale=0.0, page_size=16) -> pkv_shape:
    return pkv_shape(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim),
                     int(page_size), int(block_table_stride), int(num_pages),
                     DTYPES[dtype] if isinstance(dtype, str) else int(dtype),
                     float(sm_scale))


def make_opts(mode="auto", num_splits=0, chunk_pages=0, num_cus=0,
              queue_seed=0, merge="fused") -> pkv_opts:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    mg = MERGES[merge] if isinstance(merge, str) else int(merge)
    return pkv_opts(m, int(num_splits), int(chunk_pages), int(num_cus),
                    int(queue_seed) & 0xFFFFFFFF, mg)


_I32_ARRAY_TYPES: dict = {}


def _lens(seq_lens_host):
    """The lengths as a contiguous int32 array and a pointer to it. A
    writable contiguous int32 ndarray (what a serving loop re-plans with
    every step) is passed through its buffer without a copy; anything else
    is converted first."""
    a = seq_lens_host
    if type(a) is np.ndarray and a.dtype == np.int32 and a.flags.c_contiguous \
            and a.flags.writeable and a.size:
        t = _I32_ARRAY_TYPES.get(a.size)
        if t is None:
            t = _I32_ARRAY_TYPES[a.size] = C.c_int32 * a.size
        return a, t.from_buffer(a)
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(C.POINTER(C.c_int32))


def pkv_plan_create(shape: pkv_shape, seq_lens_host, opts: pkv_opts | None = None) -> int:
    arr, ptr = _lens(seq_lens_host)
    out = _P()
    st = LIB.pkv_plan_create(C.byref(shape), ptr if arr.size else None,
                             C.byref(opts) if opts is not None else None, C.byref(out))
    _check(st, "pkv_plan_create")
    return int(out.value)


def pkv_plan_update(plan: int, seq_lens_host) -> None:
    arr, ptr = _lens(seq_lens_host)
    _check(LIB.pkv_plan_update(plan, ptr if arr.size else None), "pkv_plan_update")


def pkv_plan_upload_needed(plan: int) -> bool:
    needed = C.c_int32(1)
    _check(LIB.pkv_plan_upload_needed(plan, C.byref(needed)), "pkv_plan_upload_needed")
    return bool(needed.value)


def pkv_plan_workspace_bytes(plan: int) -> int:
    return int(LIB.pkv_plan_workspace_bytes(plan))


def pkv_plan_upload(plan: int, workspace, workspace_bytes: int, stream=0) -> None:
    _check(LIB.pkv_plan_upload(plan, _ptr(workspace), int(workspace_bytes),
                               _ptr(stream) or None), "pkv_plan_upload")


def _struct_dict(s) -> dict:
    return {name: getattr(s, name) for name, _ in s._fields_ if name != "reserved"}


def pkv_plan_stats_get(plan: int) -> dict:
    s = pkv_plan_stats()
    _check(LIB.pkv_plan_stats_get(plan, C.byref(s)), "pkv_plan_stats_get")
    d = _struct_dict(s)
    d["mode_name"] = MODE_NAMES.get(d["mode"], str(d["mode"]))
    return d


def pkv_plan_layout_get(plan: int) -> dict:
    s = pkv_workspace_layout()
    _check(LIB.pkv_plan_layout_get(plan, C.byref(s)), "pkv_plan_layout_get")
    return _struct_dict(s)


def pkv_plan_queue_get(plan: int, batch: int, num_kv_heads: int | None = None,
                       full: bool = False):
    """Host image of the upload: (items int32 [n, 4] = {b*Hkv+g, page_begin,
    page_end, slot} (all 8 fields with ``full``), meta int32 [B, 2], counters
    int32 [B*Hkv] or empty)."""
    lay = pkv_plan_layout_get(plan)
    need = pkv_plan_stats_get(plan)["upload_bytes"]
    buf = np.zeros(max(need, 1), dtype=np.uint8)
    _check(LIB.pkv_plan_queue_get(plan, buf.ctypes.data, need), "pkv_plan_queue_get")
    img = buf[:need]

    def cut(off, nbytes):
        return img[off:off + nbytes] if off + nbytes <= need else img[:0]

    items = cut(lay["items_offset"], 32 * lay["num_items"])
    has_meta = lay["counters_offset"] > lay["meta_offset"]  # sections are packed
    meta = cut(lay["meta_offset"], 8 * batch) if has_meta else img[:0]
    rows = batch * num_kv_heads if num_kv_heads is not None else 0
    cnt = cut(lay["counters_offset"], COUNTER_STRIDE * rows)
    cnt = cnt.view(np.int32).reshape(-1, COUNTER_STRIDE // 4)[:, 0] if cnt.size else cnt
    it = items.view(np.int32).reshape(-1, 8)
    return ((it if full else it[:, :4]).copy(),
            meta.view(np.int32).reshape(-1, 2).copy(),
            cnt.view(np.int32).copy())


def pkv_decode(plan: int, q, k_pool, v_pool, block_table, seq_lens, out, stream=0) -> None:
    _check(LIB.pkv_decode(plan, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                          _ptr(seq_lens), _ptr(out), _ptr(stream) or None), "pkv_decode")


def pkv_decode_static(plan: int, q, k_pool, v_pool, block_table, seq_lens, out, stream=0) -> None:
    _check(LIB.pkv_decode_static(plan, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                 _ptr(seq_lens), _ptr(out), _ptr(stream) or None),
           "pkv_decode_static")


def pkv_decode_append(plan: int, q, k_new, v_new, k_pool, v_pool, block_table, seq_lens,
                      out, new_seq_lens=None, stream=0) -> None:
    _check(LIB.pkv_decode_append(plan, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                 _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                                 _ptr(new_seq_lens), _ptr(out), _ptr(stream) or None),
           "pkv_decode_append")


def pkv_decode_marked(plan: int, q, k_pool, v_pool, block_table, seq_lens, out, stream=0,
                      before=None, after_partial=None, after_merge=None) -> None:
    _check(LIB.pkv_decode_marked(plan, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(out),
                                 _ptr(stream) or None, _ptr(before), _ptr(after_partial),
                                 _ptr(after_merge)), "pkv_decode_marked")


def pkv_plan_destroy(plan: int) -> None:
    if plan:
        LIB.pkv_plan_destroy(plan)


def pkv_status_string(status: int) -> str:
    return LIB.pkv_status_string(int(status)).decode()


def pkv_last_error() -> str:
    return LIB.pkv_last_error().decode(errors="replace")


def pkv_version() -> int:
    return int(LIB.pkv_version())


# ------------------------------------------------------------- KV append


def _i32(arr):
    """A writable contiguous int32 numpy view and its ctypes pointer."""
    a = np.ascontiguousarray(arr, dtype=np.int32)
    return a, a.ctypes.data_as(C.POINTER(C.c_int32))


def pkv_pool_create(num_pages: int) -> int:
    h = C.c_void_p()
    _check(LIB.pkv_pool_create(int(num_pages), C.byref(h)), "pkv_pool_create")
    return h.value


def pkv_pool_destroy(pool: int) -> None:
    if pool:
        LIB.pkv_pool_destroy(pool)


def pkv_pool_free_pages(pool: int) -> int:
    return int(LIB.pkv_pool_free_pages(pool))


def pkv_pool_alloc(pool: int, n: int) -> np.ndarray:
    out, ptr = _i32(np.zeros(max(int(n), 1), dtype=np.int32))
    _check(LIB.pkv_pool_alloc(pool, int(n), ptr), "pkv_pool_alloc")
    return out[:int(n)].copy()


def pkv_pool_free(pool: int, pages) -> None:
    a, ptr = _i32(pages)
    _check(LIB.pkv_pool_free(pool, ptr, int(a.size)), "pkv_pool_free")


def pkv_append_prepare(pool: int, seq_lens_host, block_table_host: np.ndarray,
                       page_size: int = 16) -> int:
    """Host half of an append step; updates ``block_table_host`` (int32
    [B, stride], C-contiguous) in place and returns the pages taken."""
    if block_table_host.dtype != np.int32 or not block_table_host.flags.c_contiguous:
        raise ValueError("block_table_host must be a C-contiguous int32 array")
    lens, lp = _i32(seq_lens_host)
    taken = C.c_int32(0)
    _check(LIB.pkv_append_prepare(pool, int(lens.size), int(block_table_host.shape[1]),
                                  int(page_size), lp,
                                  block_table_host.ctypes.data_as(C.POINTER(C.c_int32)),
                                  C.byref(taken)), "pkv_append_prepare")
    return int(taken.value)


def pkv_pool_release_row(pool: int, block_table_row: np.ndarray, seq_len: int,
                         page_size: int = 16) -> None:
    """Return a finished row's pages; ``block_table_row`` (int32, contiguous)
    is updated in place (entries set to -1)."""
    if block_table_row.dtype != np.int32 or not block_table_row.flags.c_contiguous:
        raise ValueError("block_table_row must be a C-contiguous int32 array")
    _check(LIB.pkv_pool_release_row(pool, block_table_row.ctypes.data_as(C.POINTER(C.c_int32)),
                                    int(seq_len), int(page_size)), "pkv_pool_release_row")


def pkv_append(shape: pkv_shape, k_new, v_new, k_pool, v_pool, block_table, seq_lens,
               new_seq_lens=None, stream=0) -> None:
    _check(LIB.pkv_append(C.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                          _ptr(block_table), _ptr(seq_lens), _ptr(new_seq_lens),
                          _ptr(stream) or None), "pkv_append")


def pkv_paged_read(plan: int, k_pool, v_pool, block_table, seq_lens, sink, stream=0) -> None:
    """Read the K/V tiles ``pkv_decode`` with this plan reads, with its work
    split and load path and nothing else (measurement aid: the cost of the
    paged gather alone)."""
    _check(LIB.pkv_paged_read(plan, _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                              _ptr(seq_lens), _ptr(sink), _ptr(stream) or None), "pkv_paged_read")


def pkv_stream_read(a, b, bytes_each: int, grid: int, sink, stream=0) -> None:
    """Plain streaming read of ``bytes_each`` bytes of each of ``a`` and ``b``
    (measurement aid: the HBM ceiling of a one-pass read)."""
    _check(LIB.pkv_stream_read(_ptr(a), _ptr(b), int(bytes_each), int(grid), _ptr(sink),
                               _ptr(stream) or None), "pkv_stream_read")
