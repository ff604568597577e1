"""Python binding of the MI355X multi-LoRA apply library (liblora_mi355x.so).

Thin ctypes marshalling over the C ABI declared in include/lora.h: every
function here has the C function's name and arguments, takes tensors (or raw
integer device pointers) and the current HIP stream, and raises LoraError
when the C call returns a non-zero status.  All computation happens in the
HIP library; there is no fallback of any kind.  Importing this package fails
if the library has not been built (``python -m segmented_gathered_rank_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "LORA_F32", "LORA_BF16", "LORA_MAX_RANK", "LORA_META_WORDS", "META", "LoraError",
    "lora_segments", "lora_pool_stats_t", "LIB_PATH",
    "lora_abi_version", "lora_status_str", "lora_pool_create", "lora_pool_destroy",
    "lora_pool_load", "lora_pool_evict", "lora_pool_stats", "lora_pool_read",
    "lora_segments_bytes", "lora_segments_bind", "lora_build_segments",
    "lora_segments_check", "lora_shrink_workspace_bytes", "lora_shrink", "lora_shrink_noalloc",
    "LORA_NOALLOC_SCRATCH_BYTES",
    "lora_expand", "lora_apply_sgmv", "lora_apply_sgmv_multi", "lora_x_run", "lora_apply_bgmv", "lora_apply_bgmv_ids", "lora_apply_bgmv_packed", "lora_fused_gemm", "lora_fused_gemm_fp8w",
    "LORA_TIER_GPU", "LORA_TIER_HOST", "LORA_TIER_COLD", "lora_tiers_create", "lora_tiers_destroy",
    "lora_tiers_touch", "lora_tiers_stats", "lora_tiers_slot_of", "lora_tiers_acquire",
    "lora_tiers_batch_done", "lora_tiers_prefetch",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora_mi355x.so")

LORA_F32 = 0
LORA_BF16 = 1
LORA_MAX_RANK = 64
LORA_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024
LORA_META_WORDS = 16
META = {
    "n_seg": 0, "n_active": 1, "max_seg_len": 2, "n_bad": 3, "n_units_short": 4,
    "n_units_all": 5, "n_tiles": 6, "unit_tokens": 7, "tile_tokens": 8, "long_min": 9,
    "n_tokens": 10, "n_slots": 11,
}
STATUS = {
    0: "LORA_OK", -1: "LORA_ERR_ARG", -2: "LORA_ERR_SHAPE", -3: "LORA_ERR_RANK",
    -4: "LORA_ERR_NO_PAGES", -5: "LORA_ERR_SLOT", -6: "LORA_ERR_DTYPE", -7: "LORA_ERR_HIP",
    -8: "LORA_ERR_DEVICE_IDS", -9: "LORA_ERR_WORKSPACE",
}

try:  # load torch's HIP runtime first so that the library and torch share one runtime
    import torch  # noqa: F401
except ImportError:
    pass

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m segmented_gathered_rank_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)


class LoraError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {STATUS.get(status, status)} ({_lib.lora_status_str(status).decode()})")


class lora_segments(ctypes.Structure):
    _fields_ = [("perm", ctypes.c_void_p), ("seg_start", ctypes.c_void_p), ("seg_slot", ctypes.c_void_p),
                ("meta", ctypes.c_void_p), ("units", ctypes.c_void_p), ("tiles", ctypes.c_void_p),
                ("work", ctypes.c_void_p),
                ("n_tokens", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("max_segs", ctypes.c_int32),
                ("max_units", ctypes.c_int32), ("max_tiles", ctypes.c_int32), ("n_chunks", ctypes.c_int32)]


class lora_pool_stats_t(ctypes.Structure):
    _fields_ = [("n_pages", ctypes.c_int64), ("free_pages", ctypes.c_int64),
                ("loaded_entries", ctypes.c_int32), ("loaded_slots", ctypes.c_int32),
                ("loads", ctypes.c_int64), ("evicts", ctypes.c_int64)]


_P, _I32, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SEGP = ctypes.POINTER(lora_segments)
_SIGS = {
    "lora_abi_version": (_I32, []),
    "lora_status_str": (ctypes.c_char_p, [_I32]),
    "lora_pool_create": (_I32, [ctypes.POINTER(_P), _I32, _I32, _I64, _I64, _I32, _I32,
                                ctypes.POINTER(_I64), ctypes.POINTER(_I64), _I32]),
    "lora_pool_destroy": (_I32, [_P]),
    "lora_pool_load": (_I32, [_P, _I32, _I32, _I32, _P, _P, _F, _P]),
    "lora_pool_evict": (_I32, [_P, _I32, _P]),
    "lora_pool_stats": (_I32, [_P, ctypes.POINTER(lora_pool_stats_t)]),
    "lora_pool_read": (_I32, [_P, _I32, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_F), _P, _P,
                              ctypes.POINTER(_I32), _I32]),
    "lora_segments_bytes": (_SZ, [_I32, _I32]),
    "lora_segments_bind": (_I32, [_P, _SZ, _I32, _I32, _SEGP]),
    "lora_build_segments": (_I32, [_P, _SEGP, _P]),
    "lora_segments_check": (_I32, [_SEGP, _P, ctypes.POINTER(_I32)]),
    "lora_shrink_workspace_bytes": (_SZ, [_P, _I32, _I32]),
    "lora_shrink": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _SEGP, _P, _I64, _I64, _P, _SZ, _P]),
    "lora_shrink_noalloc": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _SEGP, _P, _I64, _I64, _P]),
    "lora_expand": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _SEGP, _P, _I64, _I64, _I32, _P]),
    "lora_apply_sgmv": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _SEGP, _P, _I64, _I64, _P, _I64, _I64, _I32,
                               _P, _SZ, _P]),
    "lora_apply_sgmv_multi": (_I32, [_P, _I32, _I32, _P, _I32, _SEGP, _P, _I64, _I64, _P, _I64, _I64, _I32,
                                     _P, _SZ, _P]),
    "lora_apply_bgmv": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _SEGP, _P, _I64, _I64, _I32, _P]),
    "lora_apply_bgmv_ids": (_I32, [_P, _I32, _I32, _P, _I64, _I64, _P, _I32, _P, _I64, _I64, _I32, _P]),
    "lora_apply_bgmv_packed": (_I32, [_P, _I32, _I32, _P, _I64, _SEGP, _P, _I64, _I64, _I32, _P]),
    "lora_fused_gemm": (_I32, [_P, _I32, _P, _I64, _P, _I64, _P, _I32, _P, _I64, _P]),
    "lora_fused_gemm_fp8w": (_I32, [_P, _I32, _P, _I64, _P, _I64, _P, _P, _I32, _P, _I64, _P]),
    "lora_tiers_create": (_I32, [ctypes.POINTER(_P), _I32, _I32]),
    "lora_tiers_destroy": (_I32, [_P]),
    "lora_tiers_touch": (_I32, [_P, _P, _I32, _P, _P, _P]),
    "lora_tiers_stats": (_I32, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "lora_tiers_slot_of": (_I32, [_P, _I32, ctypes.POINTER(_I32)]),
    "lora_tiers_acquire": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _P]),
    "lora_tiers_batch_done": (_I32, [_P, _P]),
    "lora_tiers_prefetch": (_I32, [_P, _P, _P, _I32, _P, _P, _P, ctypes.POINTER(_I32)]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


# ------------------------------------------------------------------ marshalling
def _ptr(a) -> Optional[int]:
    """Device/host address of a tensor, numpy array or integer (None -> NULL)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return int(a.data_ptr())
    if hasattr(a, "ctypes"):
        return int(a.ctypes.data)
    raise TypeError(f"cannot take the address of {type(a)!r}")


def _stream(stream) -> Optional[int]:
    """hipStream_t handle: an explicit int/stream object, else torch's current stream."""
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except Exception:  # torch missing: the null stream
            pass
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _check(status: int, call: str):
    if status != 0:
        raise LoraError(status, call)


# ------------------------------------------------------------------ the C ABI
def lora_abi_version() -> int:
    return _lib.lora_abi_version()


def lora_status_str(status: int) -> str:
    return _lib.lora_status_str(status).decode()


def lora_pool_create(device: int, wdtype: int, page_elems: int, n_pages: int, n_slots: int,
                     n_modules: int, h_in: Sequence[int], h_out: Sequence[int], max_rank: int) -> int:
    """Returns the pool handle (an integer address)."""
    if len(h_in) != n_modules or len(h_out) != n_modules:
        raise ValueError("h_in and h_out need one entry per module")
    out = _P()
    hin = (_I64 * n_modules)(*h_in)
    hout = (_I64 * n_modules)(*h_out)
    _check(_lib.lora_pool_create(ctypes.byref(out), device, wdtype, page_elems, n_pages, n_slots,
                                 n_modules, hin, hout, max_rank), "lora_pool_create")
    return out.value


def lora_pool_destroy(pool: int) -> None:
    _check(_lib.lora_pool_destroy(pool), "lora_pool_destroy")


def lora_pool_load(pool: int, slot: int, module: int, rank: int, A, B, scale: float, stream=None) -> None:
    _check(_lib.lora_pool_load(pool, slot, module, rank, _ptr(A), _ptr(B), scale, _stream(stream)),
           "lora_pool_load")


def lora_pool_evict(pool: int, slot: int, stream=None) -> None:
    _check(_lib.lora_pool_evict(pool, slot, _stream(stream)), "lora_pool_evict")


def lora_pool_stats(pool: int) -> dict:
    st = lora_pool_stats_t()
    _check(_lib.lora_pool_stats(pool, ctypes.byref(st)), "lora_pool_stats")
    return {k: getattr(st, k) for k, _ in lora_pool_stats_t._fields_}


def lora_pool_read(pool: int, slot: int, module: int, A=None, B=None, max_pages: int = 0):
    """Debug read-back into host arrays A, B (optional).  Returns (rank, scale, pages)."""
    rank, scale = _I32(), _F()
    pages = (_I32 * max(max_pages, 1))()
    _check(_lib.lora_pool_read(pool, slot, module, ctypes.byref(rank), ctypes.byref(scale), _ptr(A), _ptr(B),
                               pages if max_pages > 0 else None, max_pages), "lora_pool_read")
    return rank.value, scale.value, list(pages)[:max_pages]


def lora_segments_bytes(n_tokens: int, n_slots: int) -> int:
    return int(_lib.lora_segments_bytes(n_tokens, n_slots))


def lora_segments_bind(buf, n_tokens: int, n_slots: int, nbytes: Optional[int] = None) -> lora_segments:
    """Binds views over device buffer ``buf``; the returned struct keeps ``buf`` alive."""
    seg = lora_segments()
    if nbytes is None:
        nbytes = buf.numel() * buf.element_size()
    _check(_lib.lora_segments_bind(_ptr(buf), nbytes, n_tokens, n_slots, ctypes.byref(seg)),
           "lora_segments_bind")
    seg._buf = buf
    return seg


def lora_build_segments(ids, seg: lora_segments, stream=None) -> None:
    _check(_lib.lora_build_segments(_ptr(ids), ctypes.byref(seg), _stream(stream)), "lora_build_segments")


def lora_segments_check(seg: lora_segments, stream=None):
    """Returns (status, meta words).  Does not raise for LORA_ERR_DEVICE_IDS."""
    meta = (_I32 * LORA_META_WORDS)()
    st = _lib.lora_segments_check(ctypes.byref(seg), _stream(stream), meta)
    if st not in (0, -8):
        raise LoraError(st, "lora_segments_check")
    return st, list(meta)


def lora_shrink_workspace_bytes(pool: int, n_tokens: int, n_modules: int) -> int:
    return int(_lib.lora_shrink_workspace_bytes(pool, n_tokens, n_modules))


def lora_shrink(pool: int, module0: int, n_modules: int, x, ld_x: int, module_stride_x: int,
                seg: lora_segments, t, ld_t: int, module_stride_t: int, ws=None, ws_bytes: int = 0,
                stream=None) -> None:
    if ws is not None and ws_bytes == 0 and hasattr(ws, "numel"):
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.lora_shrink(pool, module0, n_modules, _ptr(x), ld_x, module_stride_x, ctypes.byref(seg),
                            _ptr(t), ld_t, module_stride_t, _ptr(ws), ws_bytes, _stream(stream)),
           "lora_shrink")


def lora_shrink_noalloc(pool: int, module0: int, n_modules: int, x, ld_x: int, module_stride_x: int,
                        seg: lora_segments, t, ld_t: int, module_stride_t: int, stream=None) -> None:
    _check(_lib.lora_shrink_noalloc(pool, module0, n_modules, _ptr(x), ld_x, module_stride_x, ctypes.byref(seg),
                                    _ptr(t), ld_t, module_stride_t, _stream(stream)), "lora_shrink_noalloc")


def lora_expand(pool: int, module0: int, n_modules: int, t, ld_t: int, module_stride_t: int,
                seg: lora_segments, y, ld_y: int, module_stride_y: int, ydtype: int, stream=None) -> None:
    _check(_lib.lora_expand(pool, module0, n_modules, _ptr(t), ld_t, module_stride_t, ctypes.byref(seg),
                            _ptr(y), ld_y, module_stride_y, ydtype, _stream(stream)), "lora_expand")


def lora_apply_sgmv(pool: int, module0: int, n_modules: int, x, ld_x: int, module_stride_x: int,
                    seg: lora_segments, t, ld_t: int, module_stride_t: int, y, ld_y: int, module_stride_y: int,
                    ydtype: int, ws=None, ws_bytes: int = 0, stream=None) -> None:
    if ws is not None and ws_bytes == 0 and hasattr(ws, "numel"):
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.lora_apply_sgmv(pool, module0, n_modules, _ptr(x), ld_x, module_stride_x, ctypes.byref(seg),
                                _ptr(t), ld_t, module_stride_t, _ptr(y), ld_y, module_stride_y, ydtype,
                                _ptr(ws), ws_bytes, _stream(stream)), "lora_apply_sgmv")


class lora_x_run(ctypes.Structure):
    _fields_ = [("x", _P), ("ld_x", _I64), ("module_stride_x", _I64), ("n_modules", _I32)]


def lora_apply_sgmv_multi(pool: int, module0: int, n_modules: int, runs, seg: lora_segments, t, ld_t: int,
                          module_stride_t: int, y, ld_y: int, module_stride_y: int, ydtype: int, ws=None,
                          ws_bytes: int = 0, stream=None) -> None:
    """runs: (x, ld_x, module_stride_x, n_modules) per run of consecutive modules."""
    arr = (lora_x_run * len(runs))(*[lora_x_run(_ptr(x), ld, ms, n) for (x, ld, ms, n) in runs])
    if ws is not None and ws_bytes == 0 and hasattr(ws, "numel"):
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.lora_apply_sgmv_multi(pool, module0, n_modules, arr, len(runs), ctypes.byref(seg), _ptr(t), ld_t,
                                      module_stride_t, _ptr(y), ld_y, module_stride_y, ydtype, _ptr(ws), ws_bytes,
                                      _stream(stream)), "lora_apply_sgmv_multi")


def lora_apply_bgmv(pool: int, module0: int, n_modules: int, x, ld_x: int, module_stride_x: int,
                    seg: lora_segments, y, ld_y: int, module_stride_y: int, ydtype: int,
                    stream=None) -> None:
    _check(_lib.lora_apply_bgmv(pool, module0, n_modules, _ptr(x), ld_x, module_stride_x, ctypes.byref(seg),
                                _ptr(y), ld_y, module_stride_y, ydtype, _stream(stream)), "lora_apply_bgmv")


def lora_apply_bgmv_ids(pool: int, module0: int, n_modules: int, x, ld_x: int, module_stride_x: int, ids,
                        n_tokens: int, y, ld_y: int, module_stride_y: int, ydtype: int, stream=None) -> None:
    _check(_lib.lora_apply_bgmv_ids(pool, module0, n_modules, _ptr(x), ld_x, module_stride_x, _ptr(ids), n_tokens,
                                    _ptr(y), ld_y, module_stride_y, ydtype, _stream(stream)), "lora_apply_bgmv_ids")


def lora_apply_bgmv_packed(pool: int, module0: int, n_modules: int, x, ld_x: int, seg: lora_segments, y,
                           ld_y: int, module_stride_y: int, ydtype: int, stream=None) -> None:
    _check(_lib.lora_apply_bgmv_packed(pool, module0, n_modules, _ptr(x), ld_x, ctypes.byref(seg), _ptr(y), ld_y,
                                       module_stride_y, ydtype, _stream(stream)), "lora_apply_bgmv_packed")


def lora_fused_gemm(pool: int, module: int, x, ld_x: int, w, ld_w: int, ids, n_tokens: int, y, ld_y: int,
                    stream=None) -> None:
    _check(_lib.lora_fused_gemm(pool, module, _ptr(x), ld_x, _ptr(w), ld_w, _ptr(ids), n_tokens, _ptr(y), ld_y,
                                _stream(stream)), "lora_fused_gemm")


def lora_fused_gemm_fp8w(pool: int, module: int, x, ld_x: int, w8, ld_w: int, w_scale, ids, n_tokens: int, y,
                         ld_y: int, stream=None) -> None:
    _check(_lib.lora_fused_gemm_fp8w(pool, module, _ptr(x), ld_x, _ptr(w8), ld_w, _ptr(w_scale), _ptr(ids),
                                     n_tokens, _ptr(y), ld_y, _stream(stream)), "lora_fused_gemm_fp8w")


# ------------------------------------------------------------------ adapter tiers
LORA_TIER_GPU, LORA_TIER_HOST, LORA_TIER_COLD = 0, 1, 2
LORA_FETCH_FN = ctypes.CFUNCTYPE(_I32, _P, _I32, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_F), _P, _P)


def lora_tiers_create(gpu_slots: int, host_slots: int) -> int:
    out = _P()
    _check(_lib.lora_tiers_create(ctypes.byref(out), gpu_slots, host_slots), "lora_tiers_create")
    return out.value


def lora_tiers_destroy(tiers: int) -> None:
    _check(_lib.lora_tiers_destroy(tiers), "lora_tiers_destroy")


def lora_tiers_touch(tiers: int, ids):
    """Policy only: returns (tier, slot, evicted) int32 arrays, one entry per request."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = ids.shape[0]
    tier, slot, ev = (np.empty(n, np.int32) for _ in range(3))
    _check(_lib.lora_tiers_touch(tiers, _ptr(ids), n, _ptr(tier), _ptr(slot), _ptr(ev)), "lora_tiers_touch")
    return tier, slot, ev


def lora_tiers_stats(tiers: int) -> dict:
    g, h, c = _I64(), _I64(), _I64()
    _check(_lib.lora_tiers_stats(tiers, ctypes.byref(g), ctypes.byref(h), ctypes.byref(c)), "lora_tiers_stats")
    return {"gpu_hits": g.value, "host_hits": h.value, "cold_loads": c.value}


def lora_tiers_slot_of(tiers: int, adapter: int) -> int:
    s = _I32()
    _check(_lib.lora_tiers_slot_of(tiers, adapter, ctypes.byref(s)), "lora_tiers_slot_of")
    return s.value


def lora_tiers_acquire(tiers: int, pool: int, ids, fetch, stream=None):
    """One batch through the tiers: returns the slot id of each request (int32
    array) after scheduling the uploads of GPU misses on `stream`.  fetch(adapter,
    module) -> None (no adapter for that module) or (rank, scale, A, B) with A
    [rank][h_in] and B [rank][h_out] host arrays in the pool's storage dtype
    (bf16 as uint16 bits)."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    n = ids.shape[0]
    slots = np.empty(n, np.int32)
    errors = []
    cb = _fetch_cb(fetch, errors)
    st = _lib.lora_tiers_acquire(tiers, pool, _ptr(ids), n, ctypes.cast(cb, _P), None, _ptr(slots),
                                 _stream(stream))
    if errors:
        raise errors[0]
    _check(st, "lora_tiers_acquire")
    return slots


def _fetch_cb(fetch, errors):
    import numpy as np

    def _cb(ctx, adapter, module, rank, scale, a_ptr, b_ptr):
        try:
            got = fetch(int(adapter), int(module))
            if got is None:
                rank[0] = 0
                scale[0] = 0.0
                return 0
            r, s, A, B = got
            A = np.ascontiguousarray(A)
            B = np.ascontiguousarray(B)
            ctypes.memmove(a_ptr, A.ctypes.data, A.nbytes)
            ctypes.memmove(b_ptr, B.ctypes.data, B.nbytes)
            rank[0] = int(r)
            scale[0] = float(s)
            return 0
        except Exception as e:  # reported after the call returns
            errors.append(e)
            return 1
    return LORA_FETCH_FN(_cb)


def lora_tiers_batch_done(tiers: int, stream=None) -> None:
    _check(_lib.lora_tiers_batch_done(tiers, _stream(stream)), "lora_tiers_batch_done")


def lora_tiers_prefetch(tiers: int, pool: int, ids, fetch, stream=None) -> int:
    """Uploads the non-resident adapters of ids on `stream` (a copy stream);
    returns how many were issued.  fetch as for lora_tiers_acquire."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    errors = []
    cb = _fetch_cb(fetch, errors)
    issued = _I32()
    st = _lib.lora_tiers_prefetch(tiers, pool, _ptr(ids), ids.shape[0], ctypes.cast(cb, _P), None,
                                  _stream(stream), ctypes.byref(issued))
    if errors:
        raise errors[0]
    _check(st, "lora_tiers_prefetch")
    return issued.value
