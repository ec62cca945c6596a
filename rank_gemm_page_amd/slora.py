"""ctypes binding of libslora (include/slora.h): the same entry points, by name.

Argument marshalling only: every step of the LoRA delta runs in the HIP
library.  Device buffers are passed as raw pointers (ints) or as objects with
``data_ptr()`` (torch tensors); host arrays as numpy arrays; streams as raw
``hipStream_t`` values (ints) or objects with ``cuda_stream``.  A failed call
raises ``SloraError`` carrying the status and the library's message.  The
library must have been built (``rank_gemm_page_amd.build.build()``); there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

from .build import LIB_PATH

SLORA_OK, SLORA_E_INVAL, SLORA_E_NOMEM, SLORA_E_EXIST, SLORA_E_NOENT, SLORA_E_STALE, SLORA_E_HIP = \
    0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "SLORA_OK", -1: "SLORA_E_INVAL", -2: "SLORA_E_NOMEM", -3: "SLORA_E_EXIST",
                -4: "SLORA_E_NOENT", -5: "SLORA_E_STALE", -6: "SLORA_E_HIP"}
SLORA_F32, SLORA_F16 = 0, 1
SLORA_TUNE_MFMA_MIN_TOKENS, SLORA_TUNE_GEMV_EXPAND_ELEMS, SLORA_TUNE_MFMA_EXPAND_COLS = 0, 1, 2
SLORA_MFMA_MAX_RANK = 64          # segments of higher rank always take the vector-ALU tiles
SLORA_TUNE_MFMA_SHRINK_SPLITS, SLORA_TUNE_FUSED, SLORA_TUNE_XCDS, SLORA_TUNE_TILE_ORDER = 3, 4, 5, 6
SLORA_TUNE_FWD_GROUP, SLORA_TUNE_FWD_TILE, SLORA_TUNE_SHRINK_ROWS, SLORA_TUNE_FWD_KSPLIT = 7, 8, 9, 10

EXPORTED = [
    "slora_pool_create", "slora_pool_destroy", "slora_pool_set_tuning", "slora_alloc_pages",
    "slora_free_pages", "slora_free_count", "slora_load_adapter", "slora_unload_adapter",
    "slora_adapter_image_bytes", "slora_pack_adapter", "slora_load_adapters_async",
    "slora_adapter_pages", "slora_build_segments", "slora_segments_destroy",
    "slora_segments_get_info", "slora_segments_export", "slora_segments_tiles",
    "slora_segments_upload", "slora_segments_read_error", "slora_segments_set_launch_count",
    "slora_lora_delta", "slora_lora_delta_timed", "slora_lora_shrink", "slora_lora_expand",
    "slora_lora_forward", "slora_lora_forward_timed", "slora_last_error",
    "slora_lora_delta_multi", "slora_lora_delta_multi_timed", "slora_lora_forward_noalloc",
    "slora_segments_forward_tables",
]
# include/slora_probe.h: bandwidth probes (measurement only)
EXPORTED_PROBE = ["slora_probe_read", "slora_probe_gather"]


class SloraError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("h_in", c_int32), ("h_out", c_int32), ("n_proj", c_int32),
                ("max_adapters", c_int32), ("max_rank", c_int32), ("n_classes", c_int32),
                ("reserved0", c_int32), ("n_pages", c_int64 * 2), ("class_base", c_void_p * 2),
                ("free_order", POINTER(c_int32) * 2)]


class SegmentsInfo(ctypes.Structure):
    _fields_ = [("n_tokens", c_int32), ("n_routed", c_int32), ("n_segments", c_int32),
                ("n_proj", c_int32), ("sum_rank", c_int64), ("sum_rank_tokens", c_int64),
                ("n_shrink_tiles", c_int32), ("n_expand_tiles", c_int32),
                ("n_mfma_segments", c_int32), ("n_combine_tiles", c_int32), ("meta_bytes", c_size_t),
                ("workspace_bytes", c_size_t)]


_LIB = None


def lib():
    """The loaded libslora.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        # SLORA_LIB: another build of the same library (the sanitized host build)
        path = os.environ.get("SLORA_LIB") or LIB_PATH
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with rank_gemm_page_amd.build.build()")
        L = ctypes.CDLL(path)
        P = c_void_p
        sig = {
            "slora_pool_create": (c_int32, [POINTER(PoolDesc), POINTER(P)]),
            "slora_pool_destroy": (None, [P]),
            "slora_pool_set_tuning": (c_int32, [P, c_int32, c_int64]),
            "slora_alloc_pages": (c_int32, [P, c_int32, c_int64, POINTER(c_int32)]),
            "slora_free_pages": (c_int32, [P, c_int32, c_int64, POINTER(c_int32)]),
            "slora_free_count": (c_int64, [P, c_int32]),
            "slora_load_adapter": (c_int32, [P, c_int32, c_int32, c_float, POINTER(P), POINTER(P), P]),
            "slora_unload_adapter": (c_int32, [P, c_int32]),
            "slora_adapter_image_bytes": (c_size_t, [P, c_int32]),
            "slora_pack_adapter": (c_int32, [P, c_int32, POINTER(P), POINTER(P), P, c_size_t]),
            "slora_load_adapters_async": (c_int32, [P, c_int32, POINTER(c_int32), POINTER(c_int32),
                                                    POINTER(c_float), POINTER(P), P, c_size_t, P]),
            "slora_adapter_pages": (c_int32, [P, c_int32, c_int32, POINTER(c_int32), POINTER(c_int32),
                                              POINTER(c_int32)]),
            "slora_build_segments": (c_int32, [P, c_int32, POINTER(c_int32), POINTER(P)]),
            "slora_segments_destroy": (None, [P]),
            "slora_segments_get_info": (c_int32, [P, POINTER(SegmentsInfo)]),
            "slora_segments_export": (c_int32, [P] + [POINTER(c_int32)] * 4 + [POINTER(c_float)] +
                                      [POINTER(c_int32)] * 3),
            "slora_segments_tiles": (c_int32, [P, POINTER(c_int32), POINTER(c_int32), c_size_t]),
            "slora_segments_upload": (c_int32, [P, P, c_size_t, P]),
            "slora_segments_read_error": (c_int32, [P, P, POINTER(c_int32)]),
            "slora_segments_set_launch_count": (c_int32, [P, c_int64]),
            "slora_lora_delta": (c_int32, [P, P, c_int32, P, P, P, c_size_t, P]),
            "slora_lora_delta_timed": (c_int32, [P, P, c_int32, P, P, P, c_size_t, P, P, P]),
            "slora_lora_delta_multi": (c_int32, [P, P, c_int32, POINTER(c_int32), POINTER(P), POINTER(P), P,
                                                 c_size_t, P]),
            "slora_lora_delta_multi_timed": (c_int32, [P, P, c_int32, POINTER(c_int32), POINTER(P), POINTER(P),
                                                       P, c_size_t, P, P, P]),
            "slora_lora_shrink": (c_int32, [P, P, c_int32, P, P, c_size_t, P]),
            "slora_lora_expand": (c_int32, [P, P, c_int32, P, P, c_size_t, P]),
            "slora_lora_forward": (c_int32, [P, P, c_int32, P, P, P, P, c_size_t, P]),
            "slora_lora_forward_timed": (c_int32, [P, P, c_int32, P, P, P, P, c_size_t, P, P, P]),
            "slora_last_error": (ctypes.c_char_p, []),
            "slora_lora_forward_noalloc": (c_int32, [P, P, c_int32, P, P, P, P]),
            "slora_segments_forward_tables": (c_int32, [P, POINTER(c_int32), POINTER(c_int32), c_size_t,
                                                        POINTER(c_int32), c_size_t]),
            "slora_probe_read": (c_int32, [P, c_int64, c_int32, c_int32, P, P, P, P]),
            "slora_probe_gather": (c_int32, [P, c_int64, c_int64, P, c_int64, P, c_int64, c_int64, P,
                                             c_int64, c_int32, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, fn: str):
    if status != SLORA_OK:
        raise SloraError(status, fn, lib().slora_last_error().decode())


def _ptr(obj) -> int:
    """Raw address of a device buffer: an int, or an object with data_ptr()."""
    if obj is None:
        return 0
    if isinstance(obj, int):
        return obj
    return int(obj.data_ptr())


def _stream(obj) -> int:
    if obj is None:
        return 0
    if isinstance(obj, int):
        return obj
    return int(obj.cuda_stream)


def _i32p(arr):
    return arr.ctypes.data_as(POINTER(c_int32))


def slora_last_error() -> str:
    return lib().slora_last_error().decode()


def slora_pool_create(dtype: int, h_in: int, h_out: int, n_proj: int, max_adapters: int,
                      max_rank: int, class_base, n_pages, free_order=None):
    """class_base / n_pages / free_order: one entry per page class (1 or 2)."""
    n_classes = len(n_pages)
    d = PoolDesc()
    d.dtype, d.h_in, d.h_out, d.n_proj = dtype, h_in, h_out, n_proj
    d.max_adapters, d.max_rank, d.n_classes, d.reserved0 = max_adapters, max_rank, n_classes, 0
    keep = []
    for c in range(n_classes):
        d.n_pages[c] = int(n_pages[c])
        d.class_base[c] = _ptr(class_base[c])
        fo = None if free_order is None else free_order[c]
        if fo is not None:
            fo = np.ascontiguousarray(fo, dtype=np.int32)
            if fo.shape != (int(n_pages[c]),):
                raise ValueError("free_order[c] must have n_pages[c] entries")
            keep.append(fo)
            d.free_order[c] = _i32p(fo)
    out = c_void_p()
    _check(lib().slora_pool_create(ctypes.byref(d), ctypes.byref(out)), "slora_pool_create")
    return out


def slora_pool_destroy(pool) -> None:
    lib().slora_pool_destroy(pool)


def slora_pool_set_tuning(pool, key: int, value: int) -> None:
    _check(lib().slora_pool_set_tuning(pool, key, int(value)), "slora_pool_set_tuning")


def slora_alloc_pages(pool, cls: int, n: int) -> np.ndarray:
    out = np.empty(max(int(n), 1), dtype=np.int32)
    _check(lib().slora_alloc_pages(pool, cls, int(n), _i32p(out)), "slora_alloc_pages")
    return out[:int(n)]


def slora_free_pages(pool, cls: int, ids) -> None:
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    _check(lib().slora_free_pages(pool, cls, ids.shape[0], _i32p(ids)), "slora_free_pages")


def slora_free_count(pool, cls: int) -> int:
    return int(lib().slora_free_count(pool, cls))


def slora_load_adapter(pool, adapter_id: int, rank: int, scale: float, A=None, B=None,
                       stream=None, h_in: int = None, h_out: int = None, dtype=None) -> None:
    """A, B: lists (one per projection) of host arrays h_in x rank and rank x h_out, or None."""
    if (A is None) != (B is None):
        raise ValueError("A and B must both be given or both be None")
    if A is None:
        _check(lib().slora_load_adapter(pool, adapter_id, rank, float(scale), None, None,
                                        _stream(stream)), "slora_load_adapter")
        return
    keep, a_ptrs, b_ptrs = _factor_ptrs(A, B, rank, h_in, h_out, dtype)
    _check(lib().slora_load_adapter(pool, adapter_id, rank, float(scale), a_ptrs, b_ptrs,
                                    _stream(stream)), "slora_load_adapter")


def _factor_ptrs(A, B, rank, h_in, h_out, dtype):
    """Contiguous host copies of A[p] (h_in x rank) and B[p] (rank x h_out) and
    ctypes arrays of their addresses (the copies must outlive the call)."""
    keep = []
    a_ptrs = (c_void_p * len(A))()
    b_ptrs = (c_void_p * len(B))()
    for p, (a, b) in enumerate(zip(A, B)):
        a = np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)
        b = np.ascontiguousarray(b, dtype=dtype) if dtype is not None else np.ascontiguousarray(b)
        if a.ndim != 2 or b.ndim != 2 or a.shape[1] != rank or b.shape[0] != rank:
            raise ValueError("A[p] must be h_in x rank and B[p] rank x h_out")
        if (h_in is not None and a.shape[0] != h_in) or (h_out is not None and b.shape[1] != h_out):
            raise ValueError("A[p] / B[p] do not match the pool's h_in / h_out")
        keep += [a, b]
        a_ptrs[p] = a.ctypes.data
        b_ptrs[p] = b.ctypes.data
    return keep, a_ptrs, b_ptrs


def slora_adapter_image_bytes(pool, rank: int) -> int:
    """Bytes of one adapter image of this rank (0 on a bad rank)."""
    return int(lib().slora_adapter_image_bytes(pool, rank))


def slora_pack_adapter(pool, rank: int, A, B, image, image_bytes: int,
                       h_in: int = None, h_out: int = None, dtype=None) -> None:
    """Fill the host image at `image` (an address or an object with data_ptr())."""
    if len(A) != len(B):
        raise ValueError("A and B need one entry per projection")
    keep, a_ptrs, b_ptrs = _factor_ptrs(A, B, rank, h_in, h_out, dtype)
    _check(lib().slora_pack_adapter(pool, rank, a_ptrs, b_ptrs, _ptr(image), image_bytes),
           "slora_pack_adapter")
    del keep


def slora_load_adapters_async(pool, ids, ranks, scales, images, dev_stage, dev_stage_bytes: int,
                              stream=None) -> None:
    """Queue the fetch of adapters ids[k] from pinned packed images[k] (addresses
    or objects with data_ptr()) through the device buffer dev_stage."""
    n = len(ids)
    if not (len(ranks) == len(scales) == len(images) == n):
        raise ValueError("ids, ranks, scales and images need one entry per adapter")
    ids_a = np.ascontiguousarray(ids, dtype=np.int32)
    ranks_a = np.ascontiguousarray(ranks, dtype=np.int32)
    scales_a = np.ascontiguousarray(scales, dtype=np.float32)
    img = (c_void_p * max(n, 1))(*[_ptr(m) for m in images])
    _check(lib().slora_load_adapters_async(pool, n, _i32p(ids_a), _i32p(ranks_a),
                                           scales_a.ctypes.data_as(POINTER(c_float)), img,
                                           _ptr(dev_stage), dev_stage_bytes, _stream(stream)),
           "slora_load_adapters_async")


def slora_unload_adapter(pool, adapter_id: int) -> None:
    _check(lib().slora_unload_adapter(pool, adapter_id), "slora_unload_adapter")


def slora_adapter_pages(pool, adapter_id: int, proj: int = 0, max_rank: int = 256):
    a = np.empty(max_rank, dtype=np.int32)
    b = np.empty(max_rank, dtype=np.int32)
    r = c_int32()
    _check(lib().slora_adapter_pages(pool, adapter_id, proj, _i32p(a), _i32p(b), ctypes.byref(r)),
           "slora_adapter_pages")
    return a[:r.value].copy(), b[:r.value].copy()


def slora_build_segments(pool, ids):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = c_void_p()
    _check(lib().slora_build_segments(pool, ids.shape[0], _i32p(ids) if ids.size else None,
                                      ctypes.byref(out)), "slora_build_segments")
    return out


def slora_segments_destroy(seg) -> None:
    lib().slora_segments_destroy(seg)


def slora_segments_get_info(seg) -> dict:
    info = SegmentsInfo()
    _check(lib().slora_segments_get_info(seg, ctypes.byref(info)), "slora_segments_get_info")
    return {name: getattr(info, name) for name, _ in SegmentsInfo._fields_ if name != "reserved0"}


def slora_segments_export(seg) -> dict:
    info = slora_segments_get_info(seg)
    S, T, n = info["n_segments"], info["n_routed"], info["n_proj"] * info["sum_rank"]
    out = {"perm": np.empty(max(T, 1), np.int32), "seg_start": np.empty(S + 1, np.int32),
           "seg_adapter": np.empty(max(S, 1), np.int32), "seg_rank": np.empty(max(S, 1), np.int32),
           "seg_scale": np.empty(max(S, 1), np.float32), "seg_page_off": np.empty(S + 1, np.int32),
           "a_pages": np.empty(max(n, 1), np.int32), "b_pages": np.empty(max(n, 1), np.int32)}
    _check(lib().slora_segments_export(
        seg, _i32p(out["perm"]), _i32p(out["seg_start"]), _i32p(out["seg_adapter"]),
        _i32p(out["seg_rank"]), out["seg_scale"].ctypes.data_as(POINTER(c_float)),
        _i32p(out["seg_page_off"]), _i32p(out["a_pages"]), _i32p(out["b_pages"])),
        "slora_segments_export")
    sizes = {"perm": T, "seg_start": S + 1, "seg_adapter": S, "seg_rank": S, "seg_scale": S,
             "seg_page_off": S + 1, "a_pages": n, "b_pages": n}
    return {k: v[:sizes[k]] for k, v in out.items()}


def slora_segments_tiles(seg):
    """(layout dict, records [n_tiles, stride]) as int32 arrays, in launch order."""
    info = slora_segments_get_info(seg)
    lay = np.empty(9, np.int32)
    _check(lib().slora_segments_tiles(seg, _i32p(lay), None, 0), "slora_segments_tiles")
    keys = ["n_tiles", "stride", "tokcap", "pagecap", "n_shrink", "n_expand", "hdr", "n_combine",
            "n_splits"]
    layout = dict(zip(keys, (int(v) for v in lay)))
    n, st = layout["n_tiles"], layout["stride"]
    rec = np.zeros(max(n * st, 4), np.int32)
    _check(lib().slora_segments_tiles(seg, _i32p(lay), _i32p(rec), rec.shape[0]),
           "slora_segments_tiles")
    return layout, rec[:n * st].reshape(n, st)


def slora_segments_upload(seg, dev_meta, dev_meta_bytes: int, stream=None) -> None:
    _check(lib().slora_segments_upload(seg, _ptr(dev_meta), int(dev_meta_bytes), _stream(stream)),
           "slora_segments_upload")


def slora_segments_read_error(seg, stream=None) -> int:
    flag = c_int32()
    _check(lib().slora_segments_read_error(seg, _stream(stream), ctypes.byref(flag)),
           "slora_segments_read_error")
    return int(flag.value)



def slora_segments_set_launch_count(seg, launches: int) -> None:
    _check(lib().slora_segments_set_launch_count(seg, launches), "slora_segments_set_launch_count")

def slora_lora_delta(pool, seg, proj: int, x, y, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().slora_lora_delta(pool, seg, proj, _ptr(x), _ptr(y), _ptr(workspace),
                                  int(workspace_bytes), _stream(stream)), "slora_lora_delta")


def slora_lora_delta_timed(pool, seg, proj: int, x, y, workspace, workspace_bytes: int, stream,
                           start_event: int, stop_event: int) -> None:
    """start_event / stop_event: raw hipEvent_t handles (ints)."""
    _check(lib().slora_lora_delta_timed(pool, seg, proj, _ptr(x), _ptr(y), _ptr(workspace),
                                        int(workspace_bytes), _stream(stream), start_event,
                                        stop_event), "slora_lora_delta_timed")


def _multi_args(projs, xs, ys):
    n = len(projs)
    if len(xs) != n or len(ys) != n:
        raise ValueError("one x and one y per projection")
    pj = np.ascontiguousarray(projs, dtype=np.int32)
    xa = (c_void_p * n)(*[_ptr(x) for x in xs])
    ya = (c_void_p * n)(*[_ptr(y) for y in ys])
    return n, pj, xa, ya


def slora_lora_delta_multi(pool, seg, projs, xs, ys, workspace, workspace_bytes: int, stream=None) -> None:
    """Projections projs[i] with inputs xs[i] and outputs ys[i] in one launch."""
    n, pj, xa, ya = _multi_args(projs, xs, ys)
    _check(lib().slora_lora_delta_multi(pool, seg, n, _i32p(pj), xa, ya, _ptr(workspace), int(workspace_bytes),
                                        _stream(stream)), "slora_lora_delta_multi")


def slora_lora_delta_multi_timed(pool, seg, projs, xs, ys, workspace, workspace_bytes: int, stream,
                                 start_event: int, stop_event: int) -> None:
    n, pj, xa, ya = _multi_args(projs, xs, ys)
    _check(lib().slora_lora_delta_multi_timed(pool, seg, n, _i32p(pj), xa, ya, _ptr(workspace),
                                              int(workspace_bytes), _stream(stream), start_event, stop_event),
           "slora_lora_delta_multi_timed")


def slora_lora_shrink(pool, seg, proj: int, x, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().slora_lora_shrink(pool, seg, proj, _ptr(x), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream)), "slora_lora_shrink")


def slora_lora_expand(pool, seg, proj: int, y, workspace, workspace_bytes: int, stream=None) -> None:
    _check(lib().slora_lora_expand(pool, seg, proj, _ptr(y), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream)), "slora_lora_expand")


def slora_lora_forward(pool, seg, proj: int, x, w, y, workspace, workspace_bytes: int,
                       stream=None) -> None:
    """y = x W + s (x A) B, written (base weight w: h_in x h_out fp16, row-major)."""
    _check(lib().slora_lora_forward(pool, seg, proj, _ptr(x), _ptr(w), _ptr(y), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream)), "slora_lora_forward")


def slora_lora_forward_timed(pool, seg, proj: int, x, w, y, workspace, workspace_bytes: int, stream,
                             start_event: int, stop_event: int) -> None:
    """start_event / stop_event: raw hipEvent_t handles (ints)."""
    _check(lib().slora_lora_forward_timed(pool, seg, proj, _ptr(x), _ptr(w), _ptr(y),
                                          _ptr(workspace), int(workspace_bytes), _stream(stream),
                                          start_event, stop_event), "slora_lora_forward_timed")


def slora_probe_read(src, nbytes: int, items: int, nontemporal: bool, sink, stream=None,
                     start_event=None, stop_event=None) -> None:
    _check(lib().slora_probe_read(_ptr(src), int(nbytes), int(items), int(bool(nontemporal)), _ptr(sink),
                                  _stream(stream), start_event, stop_event), "slora_probe_read")


def slora_probe_gather(arrays, items: int, sink, stream=None, start_event=None, stop_event=None) -> None:
    """arrays: one or two (base, stride_bytes, row_bytes, rows_device_int32, n_rows) tuples."""
    a0 = arrays[0]
    a1 = arrays[1] if len(arrays) > 1 else (0, 0, 0, 0, 0)
    _check(lib().slora_probe_gather(_ptr(a0[0]), int(a0[1]), int(a0[2]), _ptr(a0[3]), int(a0[4]),
                                    _ptr(a1[0]), int(a1[1]), int(a1[2]), _ptr(a1[3]), int(a1[4]),
                                    int(items), _ptr(sink), _stream(stream), start_event, stop_event),
           "slora_probe_gather")


def slora_lora_forward_noalloc(pool, seg, proj: int, x, w, y, stream=None) -> None:
    """slora_lora_forward with the library's own workspace (no caller allocation)."""
    _check(lib().slora_lora_forward_noalloc(pool, seg, proj, _ptr(x), _ptr(w), _ptr(y), _stream(stream)),
           "slora_lora_forward_noalloc")


def slora_segments_forward_tables(seg):
    """(layout dict, rb_info [n_rb, 2], stages [n_proj, n_stages, stage_words]) of slora_lora_forward."""
    lay = np.zeros(8, np.int32)
    _check(lib().slora_segments_forward_tables(seg, _i32p(lay), None, 0, None, 0),
           "slora_segments_forward_tables")
    keys = ["n_rb", "n_rb_big", "big_rows", "small_bm", "n_stages", "packed", "stage_words", "n_proj"]
    L = dict(zip(keys, (int(v) for v in lay)))
    rb = np.zeros(max(2 * L["n_rb"], 1), np.int32)
    st = np.zeros(max(L["n_proj"] * L["n_stages"] * L["stage_words"], 1), np.int32)
    _check(lib().slora_segments_forward_tables(seg, _i32p(lay), _i32p(rb), rb.size, _i32p(st), st.size),
           "slora_segments_forward_tables")
    return (L, rb[:2 * L["n_rb"]].reshape(-1, 2),
            st[:L["n_proj"] * L["n_stages"] * L["stage_words"]].reshape(L["n_proj"], L["n_stages"],
                                                                          L["stage_words"]))
