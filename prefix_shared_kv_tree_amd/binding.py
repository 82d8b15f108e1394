"""ctypes binding of libpkvt (C ABI in include/pkvt.h).

Argument marshalling only: every function has the C function's name, takes
numpy arrays for host buffers and integer device addresses (for example
``tensor.data_ptr()``) for device buffers, and raises ``PkvtError`` on a
negative status.  The library must have been built in-tree
(``python -m prefix_shared_kv_tree_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence, Tuple

import numpy as np

# PKVT_LIB selects another build of the library (the sanitizer build of the
# host code, for CPU tests); by default the in-tree libpkvt.so.
LIB_PATH = os.environ.get("PKVT_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                      "libpkvt.so")

PKVT_OK = 0
STATUS_NAMES = {
    -1: "INVALID_ARG", -2: "NO_CHUNKS", -3: "UNKNOWN_SEQ", -4: "EMPTY_SEQ",
    -5: "UNSUPPORTED_SHAPE", -6: "BUFFER_TOO_SMALL", -7: "STALE_PLAN", -8: "HIP",
    -9: "HOST_MEMORY",
}


class PkvtError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))


class Stats(C.Structure):
    _fields_ = [("capacity", C.c_int32), ("used_chunks", C.c_int32), ("free_chunks", C.c_int32),
                ("shared_chunks", C.c_int32), ("live_seqs", C.c_int32),
                ("reserved", C.c_int32 * 3)]


class PlanOpts(C.Structure):
    _fields_ = [("phase1_chunks", C.c_int32), ("phase2_chunks", C.c_int32),
                ("min_share", C.c_int32), ("workgroups", C.c_int32), ("unit_rows", C.c_int32)]


class PlanInfo(C.Structure):
    _fields_ = [("b", C.c_int32), ("phase1_items", C.c_int32), ("phase2_items", C.c_int32),
                ("waves", C.c_int32), ("workgroups", C.c_int32), ("slots", C.c_int32),
                ("merge_rows", C.c_int32), ("shared_chunks", C.c_int32),
                ("unique_tokens", C.c_int64), ("logical_tokens", C.c_int64),
                ("structure_version", C.c_int32), ("tasks", C.c_int32),
                ("phase1_split", C.c_int32), ("phase2_split", C.c_int32),
                ("wg_units", C.c_int32), ("last_update", C.c_int32), ("patches", C.c_int32),
                ("kernel", C.c_int32)]


_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_vp = C.c_void_p
_sz = C.c_size_t

# name -> argtypes (all return int32 status unless listed in _RESTYPE)
_SIGNATURES = {
    "pkvt_pool_bytes": [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(_sz)],
    "pkvt_tree_create": [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(_vp)],
    "pkvt_tree_create_ex": [C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(_vp)],
    "pkvt_tree_destroy": [_vp],
    "pkvt_tree_build": [_vp, C.c_int32, _i32p, _i64p, _i32p, _i64p],
    "pkvt_tree_append": [_vp, C.c_int32, _i32p, _i32p, _i64p],
    "pkvt_tree_remove": [_vp, C.c_int32],
    "pkvt_tree_stats": [_vp, C.POINTER(Stats)],
    "pkvt_tree_chunk_path": [_vp, C.c_int32, _i32p, C.c_int32, _i32p],
    "pkvt_tree_seq_len": [_vp, C.c_int32, _i64p],
    "pkvt_tree_chunk_refcount": [_vp, C.c_int32, _i32p],
    "pkvt_tree_chunk_fill": [_vp, C.c_int32, _i32p],
    "pkvt_tree_moves": [_vp, _i64p, _i64p, C.c_int64, _i64p],
    "pkvt_plan": [_vp, C.c_int32, _i32p, C.POINTER(PlanOpts), C.POINTER(_sz), C.POINTER(_sz)],
    "pkvt_plan_info_get": [_vp, C.POINTER(PlanInfo)],
    "pkvt_plan_blob": [_vp, _i32p, C.c_int32, _i32p],
    "pkvt_plan_upload": [_vp, _vp, _sz, _vp],
    "pkvt_attn_decode": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, C.c_float, _vp],
    "pkvt_attn_decode_ex": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, C.c_float, _vp, _vp, _vp],
    "pkvt_attn_decode_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, C.c_float, _vp],
    "pkvt_prefill_plan": [_vp, C.c_int32, _i32p, _i64p, C.POINTER(PlanOpts), C.POINTER(_sz),
                          C.POINTER(_sz)],
    "pkvt_prefill_info_get": [_vp, C.POINTER(PlanInfo)],
    "pkvt_prefill_blob": [_vp, _i32p, C.c_int32, _i32p],
    "pkvt_prefill_upload": [_vp, _vp, _sz, _vp],
    "pkvt_prefill_attn": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, C.c_float, _vp],
    "pkvt_kv_scatter": [_vp, _vp, _vp, _vp, _vp, _vp, C.c_int64, _vp],
    "pkvt_kv_scatter_host_slots": [_vp, _vp, _vp, _i64p, _vp, _vp, C.c_int64, _vp],
    "pkvt_kv_move": [_vp, _vp, _vp, _vp, _vp, C.c_int64, _vp],
    "pkvt_last_error": [],
}
_RESTYPE = {"pkvt_tree_destroy": None, "pkvt_last_error": C.c_char_p}

_lib: Optional[C.CDLL] = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libpkvt.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpkvt.so not found at {path}; build it with "
                           "`python -m prefix_shared_kv_tree_amd.build`")
    lib = C.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPE.get(name, C.c_int32)
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    return tuple(_SIGNATURES)


def _check(name: str, rc: int):
    if rc != PKVT_OK:
        raise PkvtError(name, rc, load().pkvt_last_error().decode(errors="replace"))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int64)


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


def _p64(a: np.ndarray):
    return a.ctypes.data_as(_i64p)


# ---- pool ---------------------------------------------------------------------

def pkvt_pool_bytes(n_heads: int, head_dim: int, chunk_size: int, pool_chunks: int) -> int:
    out = _sz()
    _check("pkvt_pool_bytes", load().pkvt_pool_bytes(n_heads, head_dim, chunk_size, pool_chunks,
                                                     C.byref(out)))
    return out.value


# ---- tree ---------------------------------------------------------------------

PKVT_MATCH_CHUNKS = 0
PKVT_MATCH_TOKENS = 1


def pkvt_tree_create(n_heads: int, head_dim: int, chunk_size: int, pool_chunks: int,
                     match: str = "chunks") -> int:
    """match: "chunks" (whole-chunk prefix matching) or "tokens" (token-granular,
    with node splits; pkvt_tree_create_ex)."""
    h = _vp()
    if match == "chunks":
        _check("pkvt_tree_create", load().pkvt_tree_create(n_heads, head_dim, chunk_size,
                                                           pool_chunks, C.byref(h)))
    else:
        mode = {"tokens": PKVT_MATCH_TOKENS}.get(match, -1)
        _check("pkvt_tree_create_ex", load().pkvt_tree_create_ex(n_heads, head_dim, chunk_size,
                                                                 pool_chunks, mode, C.byref(h)))
    return h.value


def pkvt_tree_destroy(tree: int) -> None:
    load().pkvt_tree_destroy(tree)


def pkvt_tree_build(tree: int, prompts: Sequence[Sequence[int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Insert prompts; returns (seq_ids int32 [n], slots int64 [total tokens])."""
    n = len(prompts)
    lens = np.array([len(p) for p in prompts], dtype=np.int64)
    offsets = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    toks = _i32(np.concatenate([np.asarray(p, dtype=np.int32) for p in prompts]) if n else
                np.zeros(0, np.int32))
    if toks.size == 0:
        toks = np.zeros(1, np.int32)
    ids = np.zeros(max(n, 1), dtype=np.int32)
    slots = np.zeros(max(int(offsets[-1]), 1), dtype=np.int64)
    _check("pkvt_tree_build", load().pkvt_tree_build(tree, n, _p32(toks), _p64(offsets),
                                                     _p32(ids), _p64(slots)))
    return ids[:n], slots[:int(offsets[-1])]


def pkvt_tree_append(tree: int, seq_ids, tokens) -> np.ndarray:
    ids = _i32(seq_ids)
    toks = _i32(tokens)
    if ids.shape != toks.shape:
        raise ValueError("seq_ids and tokens must have the same length")
    slots = np.zeros(max(ids.size, 1), dtype=np.int64)
    _check("pkvt_tree_append", load().pkvt_tree_append(tree, ids.size, _p32(ids), _p32(toks),
                                                       _p64(slots)))
    return slots[:ids.size]


def pkvt_tree_remove(tree: int, seq_id: int) -> None:
    _check("pkvt_tree_remove", load().pkvt_tree_remove(tree, int(seq_id)))


def pkvt_tree_stats(tree: int) -> dict:
    s = Stats()
    _check("pkvt_tree_stats", load().pkvt_tree_stats(tree, C.byref(s)))
    return {k: getattr(s, k) for k, _ in Stats._fields_ if k != "reserved"}


def pkvt_tree_chunk_path(tree: int, seq_id: int) -> np.ndarray:
    n = C.c_int32()
    rc = load().pkvt_tree_chunk_path(tree, int(seq_id), None, 0, C.byref(n))
    if rc not in (PKVT_OK, -6):
        _check("pkvt_tree_chunk_path", rc)
    buf = np.zeros(max(n.value, 1), dtype=np.int32)
    _check("pkvt_tree_chunk_path", load().pkvt_tree_chunk_path(tree, int(seq_id), _p32(buf),
                                                               buf.size, C.byref(n)))
    return buf[:n.value]


def pkvt_tree_seq_len(tree: int, seq_id: int) -> int:
    n = C.c_int64()
    _check("pkvt_tree_seq_len", load().pkvt_tree_seq_len(tree, int(seq_id), C.byref(n)))
    return n.value


def pkvt_tree_chunk_refcount(tree: int, chunk_id: int) -> int:
    n = C.c_int32()
    _check("pkvt_tree_chunk_refcount", load().pkvt_tree_chunk_refcount(tree, int(chunk_id),
                                                                       C.byref(n)))
    return n.value


def pkvt_tree_chunk_fill(tree: int, chunk_id: int) -> int:
    n = C.c_int32()
    _check("pkvt_tree_chunk_fill", load().pkvt_tree_chunk_fill(tree, int(chunk_id), C.byref(n)))
    return n.value


def pkvt_tree_moves(tree: int) -> Tuple[np.ndarray, np.ndarray]:
    """(src, dst) int64 slot arrays of the K/V moves of the last build."""
    n = C.c_int64()
    rc = load().pkvt_tree_moves(tree, None, None, 0, C.byref(n))
    if rc not in (PKVT_OK, -6):
        _check("pkvt_tree_moves", rc)
    src = np.zeros(max(n.value, 1), dtype=np.int64)
    dst = np.zeros(max(n.value, 1), dtype=np.int64)
    _check("pkvt_tree_moves", load().pkvt_tree_moves(tree, _p64(src), _p64(dst), src.size,
                                                     C.byref(n)))
    return src[:n.value], dst[:n.value]


# ---- plan ---------------------------------------------------------------------

def pkvt_plan(tree: int, q_order, phase1_chunks: int = 0, phase2_chunks: int = 0,
              min_share: int = 0, workgroups: int = 0, unit_rows: int = 0) -> Tuple[int, int]:
    """Plan a batch; returns (meta_bytes, workspace_bytes)."""
    q = _i32(q_order)
    opts = PlanOpts(phase1_chunks, phase2_chunks, min_share, workgroups, unit_rows)
    mb, wb = _sz(), _sz()
    _check("pkvt_plan", load().pkvt_plan(tree, q.size, _p32(q) if q.size else None,
                                         C.byref(opts), C.byref(mb), C.byref(wb)))
    return mb.value, wb.value


def pkvt_plan_info_get(tree: int) -> dict:
    s = PlanInfo()
    _check("pkvt_plan_info_get", load().pkvt_plan_info_get(tree, C.byref(s)))
    return {k: getattr(s, k) for k, _ in PlanInfo._fields_ if k != "reserved"}


def pkvt_plan_last_update(tree: int) -> int:
    """What the last pkvt_plan did: 0 lengths only, 1 patched, 2 rebuilt."""
    s = PlanInfo()
    _check("pkvt_plan_info_get", load().pkvt_plan_info_get(tree, C.byref(s)))
    return s.last_update


def pkvt_plan_blob(tree: int) -> np.ndarray:
    n = C.c_int32()
    rc = load().pkvt_plan_blob(tree, None, 0, C.byref(n))
    if rc not in (PKVT_OK, -6):
        _check("pkvt_plan_blob", rc)
    buf = np.zeros(max(n.value, 1), dtype=np.int32)
    _check("pkvt_plan_blob", load().pkvt_plan_blob(tree, _p32(buf), buf.size, C.byref(n)))
    return buf[:n.value]


def pkvt_plan_upload(tree: int, d_meta: int, meta_bytes: int, stream: int = 0) -> None:
    _check("pkvt_plan_upload", load().pkvt_plan_upload(tree, d_meta, meta_bytes, stream or None))


# ---- prefill ---------------------------------------------------------------------

def pkvt_prefill_plan(tree: int, seq_ids, q_from, phase1_chunks: int = 0,
                      workgroups: int = 0) -> Tuple[int, int]:
    """Plan a prefill; returns (meta_bytes, workspace_bytes)."""
    ids = _i32(seq_ids)
    qf = _i64(q_from)
    if ids.shape != qf.shape:
        raise ValueError("seq_ids and q_from must have the same length")
    opts = PlanOpts(phase1_chunks, 0, 0, workgroups, 0)
    mb, wb = _sz(), _sz()
    _check("pkvt_prefill_plan", load().pkvt_prefill_plan(
        tree, ids.size, _p32(ids) if ids.size else None, _p64(qf) if qf.size else None,
        C.byref(opts), C.byref(mb), C.byref(wb)))
    return mb.value, wb.value


def pkvt_prefill_info_get(tree: int) -> dict:
    s = PlanInfo()
    _check("pkvt_prefill_info_get", load().pkvt_prefill_info_get(tree, C.byref(s)))
    return {k: getattr(s, k) for k, _ in PlanInfo._fields_ if k != "reserved"}


def pkvt_prefill_blob(tree: int) -> np.ndarray:
    n = C.c_int32()
    rc = load().pkvt_prefill_blob(tree, None, 0, C.byref(n))
    if rc not in (PKVT_OK, -6):
        _check("pkvt_prefill_blob", rc)
    buf = np.zeros(max(n.value, 1), dtype=np.int32)
    _check("pkvt_prefill_blob", load().pkvt_prefill_blob(tree, _p32(buf), buf.size, C.byref(n)))
    return buf[:n.value]


def pkvt_prefill_upload(tree: int, d_meta: int, meta_bytes: int, stream: int = 0) -> None:
    _check("pkvt_prefill_upload", load().pkvt_prefill_upload(tree, d_meta, meta_bytes,
                                                             stream or None))


def pkvt_prefill_attn(tree: int, d_meta: int, q: int, k_pool: int, v_pool: int, out: int,
                      workspace: int, workspace_bytes: int, scale: float, stream: int = 0) -> None:
    _check("pkvt_prefill_attn", load().pkvt_prefill_attn(tree, d_meta, q, k_pool, v_pool, out,
                                                         workspace or None, workspace_bytes,
                                                         float(scale), stream or None))


# ---- device work ----------------------------------------------------------------

def pkvt_attn_decode(tree: int, d_meta: int, q: int, k_pool: int, v_pool: int, out: int,
                     workspace: int, workspace_bytes: int, scale: float, stream: int = 0) -> None:
    _check("pkvt_attn_decode", load().pkvt_attn_decode(tree, d_meta, q, k_pool, v_pool, out,
                                                       workspace or None, workspace_bytes,
                                                       float(scale), stream or None))


def pkvt_attn_decode_ex(tree: int, d_meta: int, q: int, k_pool: int, v_pool: int, out: int,
                        workspace: int, workspace_bytes: int, scale: float, stream: int = 0,
                        attn_start_event: int = 0, attn_end_event: int = 0) -> None:
    _check("pkvt_attn_decode_ex", load().pkvt_attn_decode_ex(
        tree, d_meta, q, k_pool, v_pool, out, workspace or None, workspace_bytes, float(scale),
        stream or None, attn_start_event or None, attn_end_event or None))


PKVT_NOALLOC_SCRATCH_BYTES = 64 << 20


def pkvt_attn_decode_noalloc(tree: int, d_meta: int, q: int, k_pool: int, v_pool: int, out: int,
                             scale: float, stream: int = 0) -> None:
    _check("pkvt_attn_decode_noalloc", load().pkvt_attn_decode_noalloc(
        tree, d_meta, q, k_pool, v_pool, out, float(scale), stream or None))


def pkvt_kv_scatter(tree: int, k_pool: int, v_pool: int, slots: int, k_new: int, v_new: int,
                    n_tokens: int, stream: int = 0) -> None:
    _check("pkvt_kv_scatter", load().pkvt_kv_scatter(tree, k_pool, v_pool, slots, k_new, v_new,
                                                     int(n_tokens), stream or None))


def pkvt_kv_move(tree: int, k_pool: int, v_pool: int, src: int, dst: int, n: int,
                 stream: int = 0) -> None:
    """src / dst: device int64 slot arrays of n moves."""
    _check("pkvt_kv_move", load().pkvt_kv_move(tree, k_pool, v_pool, src, dst, int(n),
                                               stream or None))


PKVT_INLINE_SLOTS = 256


def pkvt_kv_scatter_host_slots(tree: int, k_pool: int, v_pool: int, slots, k_new: int,
                               v_new: int, stream: int = 0) -> None:
    """slots: host int64 array (at most PKVT_INLINE_SLOTS entries)."""
    s = _i64(slots)
    _check("pkvt_kv_scatter_host_slots", load().pkvt_kv_scatter_host_slots(
        tree, k_pool, v_pool, _p64(s), k_new, v_new, int(s.size), stream or None))


def pkvt_last_error() -> str:
    return load().pkvt_last_error().decode(errors="replace")
