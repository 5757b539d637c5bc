"""Python binding of libzipage (include/zipage.h): argument marshalling only.

Every step of the compression runs in the HIP kernels of libzipage.so; this
module only converts torch tensors and host arrays into the C structs and
pointers of the C ABI. If the library is not built, importing works but every
call raises ZipageError -- there is no fallback implementation.

Names follow the C entry points: zp_compress, zp_update_global,
zp_paged_decode, zp_compress_workspace_bytes, zp_workspace_error, plus the
BlockManager class over zp_bm_* and the timing helpers.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ZIPAGE_LIB selects another build of the library (the host-only sanitizer
# build of host_sanitize.py); by default the in-tree libzipage.so
LIB_PATH = os.environ.get("ZIPAGE_LIB") or os.path.join(HERE, "libzipage.so")

ZP_OK = 0
ZP_EINVAL = -1
ZP_EUNSUPPORTED = -2
ZP_EWORKSPACE = -3
ZP_ENOSPACE = -4
ZP_EHIP = -5
ZP_EDEVICE = -6
ZP_ESYNC = -7

ZP_F32 = 0
ZP_BF16 = 1

ZP_NONCAUSAL = 1 << 0
ZP_PROTECT_WINDOW = 1 << 1
ZP_WINDOW_RING = 1 << 2
ZP_UPDATE_GLOBAL = 1 << 3
ZP_SPLIT_UNITS = 1 << 4

ZP_KERNEL_COMPRESS = 0
ZP_KERNEL_GLOBAL = 1
ZP_KERNEL_DECODE = 2
ZP_KERNEL_CAPTURE = 3
ZP_KERNEL_REDUNDANCY_FULL = 4
ZP_KERNEL_KINDS = 5

ZP_DECODE_STATIC_BYTES = 64 << 20
KERNEL_NAMES = ("compress", "global_update", "paged_decode", "capture",
                "redundancy_full")

EXPORTED = (
    "zp_compress_workspace_bytes", "zp_compress", "zp_update_global",
    "zp_workspace_error", "zp_paged_decode", "zp_paged_decode_append",
    "zp_decode_workspace_bytes", "zp_paged_decode_split", "zp_paged_decode_split_static",
    "zp_capture_queries",
    "zp_redundancy_full",
    "zp_sched_create", "zp_sched_destroy", "zp_sched_block_manager",
    "zp_sched_add_prefix", "zp_sched_submit", "zp_sched_step", "zp_sched_complete",
    "zp_sched_get_stats",
    "zp_bm_create", "zp_bm_destroy",
    "zp_bm_alloc", "zp_bm_incref", "zp_bm_release", "zp_bm_free_count",
    "zp_bm_refcount", "zp_bm_free_list", "zp_bm_plan_compress",
    "zp_bm_commit", "zp_bm_abort", "zp_plan_freed", "zp_plan_targets",
    "zp_timing_enable", "zp_timing_read", "zp_status_str", "zp_last_error",
    "zp_version",
)


class ZipageError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str = ""):
        self.status = status
        super().__init__(f"{where}: {_status_name(status)}: {msg}")


class KVPool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("n_max", ctypes.c_int32), ("window", ctypes.c_int32),
                ("q_heads", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("w_attn", ctypes.c_float), ("w_global", ctypes.c_float),
                ("w_red", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("flags", ctypes.c_uint32)]


class BatchStruct(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("n_cap", ctypes.c_int32),
                ("slot", ctypes.c_void_p), ("n_tokens", ctypes.c_void_p),
                ("src_table", ctypes.c_void_p), ("dst_table", ctypes.c_void_p),
                ("n_pinned", ctypes.c_void_p), ("seq_pos", ctypes.c_void_p)]


class CompressOut(ctypes.Structure):
    _fields_ = [("keep_idx", ctypes.c_void_p), ("attn", ctypes.c_void_p),
                ("red", ctypes.c_void_p), ("score", ctypes.c_void_p),
                ("first_hole", ctypes.c_void_p)]


_lib = None


def _status_name(status: int) -> str:
    names = {0: "ZP_OK", -1: "ZP_EINVAL", -2: "ZP_EUNSUPPORTED",
             -3: "ZP_EWORKSPACE", -4: "ZP_ENOSPACE", -5: "ZP_EHIP",
             -6: "ZP_EDEVICE", -7: "ZP_ESYNC"}
    return names.get(status, f"status {status}")


def lib() -> ctypes.CDLL:
    """The loaded libzipage.so (raises ZipageError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ZipageError(ZP_EHIP, "load",
                          f"{LIB_PATH} is not built (run "
                          "python -m kv_cache_compression_paged_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, U = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "zp_compress_workspace_bytes": (I32, [P, P, I32, P]),
        "zp_compress": (I32, [P, P, P, P, P, P, P, U, P]),
        "zp_update_global": (I32, [P, P, P, P, P, P]),
        "zp_workspace_error": (I32, [P, P, P]),
        "zp_paged_decode": (I32, [P, P, P, P, I32, P, I32, P, P]),
        "zp_capture_queries": (I32, [P, P, P, P, I32, I32, I32, I32, P, P]),
        "zp_redundancy_full": (I32, [P, P, P, P, P, P, U, P]),
        "zp_sched_create": (P, [P]),
        "zp_sched_destroy": (None, [P]),
        "zp_sched_block_manager": (P, [P]),
        "zp_sched_add_prefix": (I32, [P, I32, P, P]),
        "zp_sched_submit": (I32, [P, I32, I32, I32, I32]),
        "zp_sched_step": (I32, [P, P]),
        "zp_sched_complete": (I32, [P]),
        "zp_sched_get_stats": (I32, [P, P]),
        "zp_paged_decode_append": (I32, [P, P, P, P, P, P, I32, P, I32, P, P]),
        "zp_decode_workspace_bytes": (I32, [P, P, I32, I32, P]),
        "zp_paged_decode_split": (I32, [P, P, P, P, P, P, I32, P, I32, P, I32, P, U, P]),
        "zp_paged_decode_split_static": (I32, [P, P, P, P, P, P, I32, P, I32, P, I32, P]),
        "zp_bm_create": (P, [I32]),
        "zp_bm_destroy": (None, [P]),
        "zp_bm_alloc": (I32, [P, I32, P]),
        "zp_bm_incref": (I32, [P, I32]),
        "zp_bm_release": (I32, [P, I32, P]),
        "zp_bm_free_count": (I32, [P]),
        "zp_bm_refcount": (I32, [P, I32]),
        "zp_bm_free_list": (I32, [P, P, I32]),
        "zp_bm_plan_compress": (I32, [P, I32, P, I32, P, I32, I32, P, P, P]),
        "zp_bm_commit": (I32, [P, P]),
        "zp_bm_abort": (I32, [P, P]),
        "zp_plan_freed": (I32, [P, P, I32]),
        "zp_plan_targets": (I32, [P, P, I32]),
        "zp_timing_enable": (I32, [I32]),
        "zp_timing_read": (I32, [P, P]),
        "zp_status_str": (ctypes.c_char_p, [I32]),
        "zp_last_error": (ctypes.c_char_p, []),
        "zp_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        # every symbol is present in the built library (a CPU test checks
        # it); a host-only build (see host_sanitize.py) has the host calls
        fn = getattr(L, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().zp_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != ZP_OK:
        raise ZipageError(status, where, last_error())


# ------------------------------------------------------------ torch glue ---

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libzipage must be contiguous")
    return t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ZP_BF16
    if t.dtype == torch.float32:
        return ZP_F32
    raise ValueError(f"unsupported element type {t.dtype}")


def _stream_handle(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_pool(k_pool, v_pool) -> KVPool:
    """KVPool struct for two tensors [layers][blocks][kv_heads][b][d]."""
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype:
        raise ValueError("k and v pools must match")
    L, nb, hkv, b, d = k_pool.shape
    return KVPool(_ptr(k_pool), _ptr(v_pool), nb, L, hkv, b, d,
                  _dtype_code(k_pool))


def make_params(n_max: int, window: int, q_heads: int, q_dtype: int,
                w_attn: float = 1.0, w_global: float = 0.5, w_red: float = 0.5,
                sm_scale: float = 0.0, flags: int = 0) -> Params:
    return Params(n_max, window, q_heads, q_dtype, w_attn, w_global, w_red,
                  sm_scale, flags)


@dataclass
class DeviceBatch:
    """Device arrays of one compression call (int32 torch tensors)."""
    slot: object
    n_tokens: object
    src_table: object          # [R][max_blocks]
    dst_table: object          # [R][n_max]
    n_pinned: object
    num_slots: int
    n_cap: int
    seq_pos: object = None     # [R] int32, ring position base (ZP_WINDOW_RING)

    def struct(self) -> BatchStruct:
        R, mb = self.src_table.shape
        return BatchStruct(R, mb, self.num_slots, self.n_cap, _ptr(self.slot),
                           _ptr(self.n_tokens), _ptr(self.src_table),
                           _ptr(self.dst_table), _ptr(self.n_pinned),
                           _ptr(self.seq_pos))


@dataclass
class Outputs:
    keep_idx: object           # [U][k] int32
    attn: object               # [U][n_cap] fp32
    red: object = None
    score: object = None
    first_hole: object = None

    def struct(self) -> CompressOut:
        return CompressOut(_ptr(self.keep_idx), _ptr(self.attn), _ptr(self.red),
                           _ptr(self.score), _ptr(self.first_hole))


def alloc_outputs(units: int, k: int, n_cap: int, device, debug: bool = False
                  ) -> Outputs:
    import torch
    o = Outputs(keep_idx=torch.empty((units, k), dtype=torch.int32, device=device),
                attn=torch.empty((units, n_cap), dtype=torch.float32, device=device),
                first_hole=torch.empty((units,), dtype=torch.int32, device=device))
    if debug:
        o.red = torch.empty((units, n_cap), dtype=torch.float32, device=device)
        o.score = torch.empty((units, n_cap), dtype=torch.float32, device=device)
    return o


def zp_compress_workspace_bytes(pool: KVPool, params: Params, num_reqs: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().zp_compress_workspace_bytes(ctypes.byref(pool),
                                             ctypes.byref(params), num_reqs,
                                             ctypes.byref(out)),
           "zp_compress_workspace_bytes")
    return out.value


def alloc_workspace(pool: KVPool, params: Params, num_reqs: int, device):
    import torch
    nbytes = zp_compress_workspace_bytes(pool, params, num_reqs)
    ws = torch.zeros((nbytes + 255) // 256 * 64, dtype=torch.int32, device=device)
    return ws


def zp_compress(pool: KVPool, batch: DeviceBatch, q_window, global_scores,
                params: Params, out: Outputs, workspace, stream=None) -> None:
    b = batch.struct()
    o = out.struct()
    _check(lib().zp_compress(ctypes.byref(pool), ctypes.byref(b), _ptr(q_window),
                             _ptr(global_scores), ctypes.byref(params),
                             ctypes.byref(o), _ptr(workspace),
                             workspace.numel() * workspace.element_size(),
                             _stream_handle(stream)), "zp_compress")


def zp_update_global(global_scores, pool: KVPool, batch: DeviceBatch,
                     out: Outputs, params: Params, stream=None) -> None:
    b = batch.struct()
    o = out.struct()
    _check(lib().zp_update_global(_ptr(global_scores), ctypes.byref(pool),
                                  ctypes.byref(b), ctypes.byref(o),
                                  ctypes.byref(params), _stream_handle(stream)),
           "zp_update_global")


def zp_workspace_error(workspace, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().zp_workspace_error(_ptr(workspace), _stream_handle(stream),
                                    ctypes.byref(code)), "zp_workspace_error")
    return code.value


def zp_paged_decode(out, q, pool: KVPool, block_tables, seq_lens,
                    params: Params, stream=None) -> None:
    R, mb = block_tables.shape
    _check(lib().zp_paged_decode(_ptr(out), _ptr(q), ctypes.byref(pool),
                                 _ptr(block_tables), mb, _ptr(seq_lens), R,
                                 ctypes.byref(params), _stream_handle(stream)),
           "zp_paged_decode")


def zp_paged_decode_append(out, q, k_new, v_new, pool: KVPool, block_tables,
                           seq_lens, params: Params, stream=None) -> None:
    R, mb = block_tables.shape
    _check(lib().zp_paged_decode_append(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                        ctypes.byref(pool), _ptr(block_tables), mb,
                                        _ptr(seq_lens), R, ctypes.byref(params),
                                        _stream_handle(stream)), "zp_paged_decode_append")


def zp_decode_workspace_bytes(pool: KVPool, params: Params, num_reqs: int,
                              splits: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().zp_decode_workspace_bytes(ctypes.byref(pool), ctypes.byref(params),
                                           num_reqs, splits, ctypes.byref(out)),
           "zp_decode_workspace_bytes")
    return out.value


def zp_paged_decode_split(out, q, pool: KVPool, block_tables, seq_lens,
                          params: Params, splits: int, workspace, k_new=None,
                          v_new=None, stream=None) -> None:
    R, mb = block_tables.shape
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().zp_paged_decode_split(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                       ctypes.byref(pool), _ptr(block_tables), mb,
                                       _ptr(seq_lens), R, ctypes.byref(params), splits,
                                       _ptr(workspace), nbytes, _stream_handle(stream)),
           "zp_paged_decode_split")


def zp_paged_decode_split_static(out, q, pool: KVPool, block_tables, seq_lens,
                                 params: Params, splits: int, k_new=None, v_new=None,
                                 stream=None) -> None:
    """Split-K decode with the partials in the library's static device
    scratch (no workspace argument; see include/zipage.h)."""
    R, mb = block_tables.shape
    _check(lib().zp_paged_decode_split_static(_ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new),
                                              ctypes.byref(pool), _ptr(block_tables), mb,
                                              _ptr(seq_lens), R, ctypes.byref(params),
                                              splits, _stream_handle(stream)),
           "zp_paged_decode_split_static")


def zp_redundancy_full(red_block, pool: KVPool, batch: DeviceBatch, params: Params,
                       workspace, red_all=None, stream=None) -> None:
    b = batch.struct()
    _check(lib().zp_redundancy_full(_ptr(red_block), _ptr(red_all), ctypes.byref(pool),
                                    ctypes.byref(b), ctypes.byref(params), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_handle(stream)), "zp_redundancy_full")


def zp_capture_queries(q_window, q, slot, pos, params: Params,
                       stream=None) -> None:
    """q_window [slots][L][w][Hq][d], q [R][L][Hq][d] (same dtype), slot and
    pos [R] int32 device tensors."""
    S, L = q_window.shape[0], q_window.shape[1]
    R = q.shape[0]
    _check(lib().zp_capture_queries(_ptr(q_window), _ptr(q), _ptr(slot), _ptr(pos),
                                    R, L, S, q.shape[-1], ctypes.byref(params),
                                    _stream_handle(stream)), "zp_capture_queries")


def timing_enable(on: bool) -> None:
    _check(lib().zp_timing_enable(1 if on else 0), "zp_timing_enable")


def timing_read() -> dict:
    n = (ctypes.c_int32 * ZP_KERNEL_KINDS)()
    ms = (ctypes.c_double * ZP_KERNEL_KINDS)()
    _check(lib().zp_timing_read(n, ms), "zp_timing_read")
    return {KERNEL_NAMES[i]: (int(n[i]), float(ms[i]))
            for i in range(ZP_KERNEL_KINDS)}


# -------------------------------------------------------- block manager ---

def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Plan:
    def __init__(self, handle, dst_tables: np.ndarray, n_pinned: np.ndarray):
        self.handle = handle
        self.dst_tables = dst_tables
        self.n_pinned = n_pinned

    def freed(self) -> List[int]:
        n = lib().zp_plan_freed(self.handle, None, 0)
        buf = np.zeros(max(n, 1), dtype=np.int32)
        lib().zp_plan_freed(self.handle, _np_ptr(buf), n)
        return buf[:n].tolist()

    def targets(self) -> List[int]:
        n = lib().zp_plan_targets(self.handle, None, 0)
        buf = np.zeros(max(n, 1), dtype=np.int32)
        lib().zp_plan_targets(self.handle, _np_ptr(buf), n)
        return buf[:n].tolist()


class BlockManager:
    """Host free list + reference counts (zp_bm_*)."""

    def __init__(self, num_blocks: int):
        self.h = lib().zp_bm_create(num_blocks)
        if not self.h:
            raise ZipageError(ZP_EINVAL, "zp_bm_create", last_error())
        self.num_blocks = num_blocks

    def __del__(self):
        h = getattr(self, "h", None)
        if h and _lib is not None:
            _lib.zp_bm_destroy(h)
            self.h = None

    def alloc(self, n: int) -> List[int]:
        buf = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib().zp_bm_alloc(self.h, n, _np_ptr(buf)), "zp_bm_alloc")
        return buf[:n].tolist()

    def incref(self, bid: int) -> None:
        _check(lib().zp_bm_incref(self.h, bid), "zp_bm_incref")

    def release(self, ids: Sequence[int]) -> None:
        a = _i32(ids)
        _check(lib().zp_bm_release(self.h, len(a), _np_ptr(a)), "zp_bm_release")

    def free_count(self) -> int:
        return lib().zp_bm_free_count(self.h)

    def refcount(self, bid: int) -> int:
        return lib().zp_bm_refcount(self.h, bid)

    def free_list(self) -> List[int]:
        n = self.free_count()
        buf = np.zeros(max(n, 1), dtype=np.int32)
        lib().zp_bm_free_list(self.h, _np_ptr(buf), n)
        return buf[:n].tolist()

    def plan_compress(self, tables, n_tokens, n_max: int, block_size: int
                      ) -> Plan:
        t = _i32(tables)
        if t.ndim != 2:
            raise ValueError("tables must be [R][max_blocks]")
        R, mb = t.shape
        nt = _i32(n_tokens)
        dst = np.zeros((R, n_max), dtype=np.int32)
        pin = np.zeros(R, dtype=np.int32)
        handle = ctypes.c_void_p()
        _check(lib().zp_bm_plan_compress(self.h, R, _np_ptr(t), mb, _np_ptr(nt),
                                         n_max, block_size, _np_ptr(dst),
                                         _np_ptr(pin), ctypes.byref(handle)),
               "zp_bm_plan_compress")
        return Plan(handle, dst, pin)

    def commit(self, plan: Plan) -> None:
        _check(lib().zp_bm_commit(self.h, plan.handle), "zp_bm_commit")
        plan.handle = None

    def abort(self, plan: Plan) -> None:
        _check(lib().zp_bm_abort(self.h, plan.handle), "zp_bm_abort")
        plan.handle = None


class SchedConfig(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("num_blocks", "block_size", "n_max", "window", "query_slots",
                 "max_running", "max_blocks")]


_PI = ctypes.POINTER(ctypes.c_int32)


class SchedPlanStruct(ctypes.Structure):
    _fields_ = [("restricted", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("num_admit", ctypes.c_int32),
                ("admit_id", _PI), ("admit_len", _PI), ("admit_slot", _PI),
                ("admit_table", _PI), ("admit_shared", _PI),
                ("num_new_slots", ctypes.c_int32), ("new_slot", _PI),
                ("num_decode", ctypes.c_int32),
                ("decode_id", _PI), ("decode_slot", _PI), ("decode_len", _PI),
                ("decode_pos", _PI), ("decode_table", _PI),
                ("num_compress", ctypes.c_int32),
                ("compress_id", _PI), ("compress_slot", _PI), ("compress_len", _PI),
                ("compress_pos", _PI), ("compress_src", _PI), ("compress_dst", _PI),
                ("compress_pinned", _PI),
                ("num_preempt", ctypes.c_int32), ("preempt_id", _PI)]


class SchedStatsStruct(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("steps", "tokens", "compressions", "preemptions", "restricted_steps",
                 "admitted", "finished")] + \
               [(n, ctypes.c_int32) for n in ("running", "waiting", "free_blocks")]


@dataclass
class SchedPlan:
    """One planned step, copied out of the scheduler (numpy int32 arrays;
    table rows padded with -1)."""
    restricted: bool
    admit_id: np.ndarray
    admit_len: np.ndarray
    admit_slot: np.ndarray
    admit_table: np.ndarray       # [A][max_blocks]
    admit_shared: np.ndarray
    new_slot: np.ndarray
    decode_id: np.ndarray
    decode_slot: np.ndarray
    decode_len: np.ndarray
    decode_pos: np.ndarray
    decode_table: np.ndarray      # [D][max_blocks]
    compress_id: np.ndarray
    compress_slot: np.ndarray
    compress_len: np.ndarray
    compress_pos: np.ndarray
    compress_src: np.ndarray      # [C][max_blocks]
    compress_dst: np.ndarray      # [C][n_max]
    compress_pinned: np.ndarray
    preempt_id: np.ndarray


def _arr(ptr, n, shape=None) -> np.ndarray:
    if n == 0:
        return np.zeros(shape if shape else (0,), dtype=np.int32)
    a = np.ctypeslib.as_array(ptr, shape=(n,)).copy()
    return a.reshape(shape) if shape else a


class Scheduler:
    """Hybrid compression/decode scheduler of the library (host only)."""

    def __init__(self, num_blocks: int, block_size: int, n_max: int, window: int,
                 query_slots: int, max_running: int, max_blocks: int):
        self.cfg = SchedConfig(num_blocks, block_size, n_max, window, query_slots,
                               max_running, max_blocks)
        h = lib().zp_sched_create(ctypes.byref(self.cfg))
        if not h:
            raise ZipageError(ZP_EINVAL, "zp_sched_create",
                              lib().zp_last_error().decode())
        self.h = h

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.zp_sched_destroy(self.h)
            self.h = None

    def add_prefix(self, blocks: int):
        group = ctypes.c_int32(0)
        ids = np.zeros(blocks, dtype=np.int32)
        _check(lib().zp_sched_add_prefix(self.h, blocks, ctypes.byref(group),
                                         _np_ptr(ids)), "zp_sched_add_prefix")
        return group.value, ids

    def submit(self, req_id: int, prompt_len: int, gen_len: int, group: int = -1) -> None:
        _check(lib().zp_sched_submit(self.h, req_id, prompt_len, gen_len, group),
               "zp_sched_submit")

    def step(self) -> SchedPlan:
        p = SchedPlanStruct()
        _check(lib().zp_sched_step(self.h, ctypes.byref(p)), "zp_sched_step")
        mb, nm = self.cfg.max_blocks, self.cfg.n_max
        A, D, C = p.num_admit, p.num_decode, p.num_compress
        return SchedPlan(
            bool(p.restricted),
            _arr(p.admit_id, A), _arr(p.admit_len, A), _arr(p.admit_slot, A),
            _arr(p.admit_table, A * mb, (A, mb)), _arr(p.admit_shared, A),
            _arr(p.new_slot, p.num_new_slots),
            _arr(p.decode_id, D), _arr(p.decode_slot, D), _arr(p.decode_len, D),
            _arr(p.decode_pos, D), _arr(p.decode_table, D * mb, (D, mb)),
            _arr(p.compress_id, C), _arr(p.compress_slot, C), _arr(p.compress_len, C),
            _arr(p.compress_pos, C), _arr(p.compress_src, C * mb, (C, mb)),
            _arr(p.compress_dst, C * nm, (C, nm)), _arr(p.compress_pinned, C),
            _arr(p.preempt_id, p.num_preempt))

    def complete(self) -> None:
        _check(lib().zp_sched_complete(self.h), "zp_sched_complete")

    def stats(self) -> dict:
        st = SchedStatsStruct()
        _check(lib().zp_sched_get_stats(self.h, ctypes.byref(st)), "zp_sched_get_stats")
        return {name: int(getattr(st, name)) for name, _ in st._fields_}

    def refcount(self, block: int) -> int:
        return int(lib().zp_bm_refcount(lib().zp_sched_block_manager(self.h), block))


def version() -> str:
    return lib().zp_version().decode()


__all__: Tuple[str, ...] = (
    "ZipageError", "KVPool", "Params", "BatchStruct", "CompressOut", "lib",
    "make_pool", "make_params", "DeviceBatch", "Outputs", "alloc_outputs",
    "alloc_workspace", "zp_compress_workspace_bytes", "zp_compress",
    "zp_update_global", "zp_workspace_error", "zp_paged_decode",
    "zp_capture_queries", "zp_paged_decode_append", "zp_decode_workspace_bytes",
    "zp_paged_decode_split", "zp_paged_decode_split_static", "zp_redundancy_full",
    "Scheduler", "SchedPlan",
    "timing_enable", "timing_read", "BlockManager", "Plan", "version",
    "EXPORTED",
)
