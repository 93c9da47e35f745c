"""ctypes declarations of libmagi_bca.so (the C ABI in include/magi_bca.h).

Loading fails loudly: there is no fallback implementation.  Build the
library first (``python -m block_causal_attention_amd.build``).
"""
from __future__ import annotations

import ctypes as C
import os

# MAGI_BCA_LIBRARY names another build of the same library (the host-
# sanitized one the CPU tests make); by default the in-tree build is loaded
LIB_PATH = os.environ.get("MAGI_BCA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libmagi_bca.so")

MAGI_OK = 0
MAGI_ERR_INVALID_ARG = -1
MAGI_ERR_UNSUPPORTED = -2
MAGI_ERR_BUFFER_TOO_SMALL = -3
MAGI_ERR_OVERLAP = -4
MAGI_ERR_HIP = -5
MASK_FULL = 0
MASK_CAUSAL = 1
MASK_INVCAUSAL = 2
MASK_BICAUSAL = 3
DTYPE_BF16 = 0
DTYPE_FP32 = 1

STATUS_NAMES = {0: "MAGI_OK", -1: "MAGI_ERR_INVALID_ARG", -2: "MAGI_ERR_UNSUPPORTED",
                -3: "MAGI_ERR_BUFFER_TOO_SMALL", -4: "MAGI_ERR_OVERLAP", -5: "MAGI_ERR_HIP"}

EXPORTS = ("magi_version", "magi_last_error", "magi_slices_build", "magi_default_tile_q",
           "magi_schedule", "magi_qknorm_rope", "magi_ffa_fwd", "magi_ffa_fwd_timed", "magi_ffa_fwd_qknorm",
           "magi_default_tile_k", "magi_schedule_kv", "magi_ffa_bwd", "magi_ffa_bwd_noalloc", "magi_slices_cross", "magi_slices_ring",
           "magi_slices_window")


class AttnSlice(C.Structure):
    _fields_ = [("q_start", C.c_int32), ("q_end", C.c_int32), ("k_start", C.c_int32),
                ("k_end", C.c_int32), ("mask_type", C.c_int32)]


class WorkItem(C.Structure):
    _fields_ = [("q_start", C.c_int32), ("q_len", C.c_int32), ("slice_begin", C.c_int32),
                ("slice_end", C.c_int32), ("kv_group", C.c_int32), ("cost", C.c_int32)]


class RingDesc(C.Structure):
    _fields_ = [("chunk_len", C.c_int32), ("ring_slots", C.c_int32), ("first_chunk", C.c_int32),
                ("num_chunks", C.c_int32), ("num_inflight", C.c_int32), ("q_offset", C.c_int32),
                ("k_offset", C.c_int32), ("kv_range", C.POINTER(C.c_int32))]


class KvReduce(C.Structure):
    _fields_ = [("key_start", C.c_int32), ("key_len", C.c_int32), ("kv_group", C.c_int32),
                ("slot_begin", C.c_int32), ("slot_count", C.c_int32)]


class CrossDesc(C.Structure):
    _fields_ = [("q_offset", C.c_int32), ("q_len", C.c_int32), ("k_offset", C.c_int32), ("k_len", C.c_int32)]


class WindowDesc(C.Structure):
    _fields_ = [("len", C.c_int32), ("window", C.c_int32), ("q_offset", C.c_int32), ("k_offset", C.c_int32)]


class SeqDesc(C.Structure):
    _fields_ = [("chunk_len", C.c_int32), ("num_kv_chunks", C.c_int32), ("num_q_chunks", C.c_int32),
                ("q_offset", C.c_int32), ("k_offset", C.c_int32), ("kv_range", C.POINTER(C.c_int32))]


class MagiError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_causal_attention_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        i32, i64, vp = C.c_int32, C.c_int64, C.c_void_p
        fp = C.POINTER(C.c_float)
        L.magi_version.restype = C.c_char_p
        L.magi_last_error.restype = C.c_char_p
        L.magi_slices_build.argtypes = [C.POINTER(SeqDesc), i32, C.POINTER(AttnSlice), i32, C.POINTER(i32)]
        L.magi_default_tile_q.argtypes = [i32, i32, i32, i32]
        L.magi_schedule.argtypes = [C.POINTER(AttnSlice), i32, i64, i64, i32, i32, i32, i32, i32,
                                    C.POINTER(WorkItem), i32, C.POINTER(i32), C.POINTER(i32), i32,
                                    C.POINTER(i32)]
        L.magi_qknorm_rope.argtypes = [vp, vp, i64, i32, i64, vp, vp, i64, i32, i64, i64, i64, vp, vp,
                                       i32, i32, vp, vp, i32, C.c_float, vp, vp, vp, C.c_float, C.c_float,
                                       vp, vp]
        L.magi_ffa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, i64, i64, i64, i64,
                                   C.c_float, vp, vp, i32, vp, i32, vp, i32, vp]
        L.magi_ffa_fwd_timed.argtypes = L.magi_ffa_fwd.argtypes + [vp, vp]
        L.magi_ffa_fwd_qknorm.argtypes = L.magi_ffa_fwd.argtypes[:-1] + [vp, i32, C.c_float, vp, vp, C.c_float,
                                                                         vp, i64, vp]
        L.magi_default_tile_k.argtypes = [i32, i32, i32, i32]
        L.magi_slices_cross.argtypes = [C.POINTER(CrossDesc), i32, C.POINTER(AttnSlice), i32, C.POINTER(i32)]
        L.magi_slices_ring.argtypes = [C.POINTER(RingDesc), C.POINTER(AttnSlice), i32, C.POINTER(i32)]
        L.magi_slices_window.argtypes = [C.POINTER(WindowDesc), i32, C.POINTER(AttnSlice), i32, C.POINTER(i32)]
        L.magi_schedule_kv.argtypes = L.magi_schedule.argtypes + [C.POINTER(i32), C.POINTER(KvReduce), i32,
                                                                   C.POINTER(i32), C.POINTER(i32)]
        L.magi_ffa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32,
                                   i64, i64, i64, i64, C.c_float, vp, i32, vp, i32, vp, i32, vp, i32, vp, i32,
                                   vp, vp, i32, i32, vp, i64, vp]
        # magi_ffa_bwd without delta (after dv) and without partial, partial_floats
        bw = L.magi_ffa_bwd.argtypes
        L.magi_ffa_bwd_noalloc.argtypes = bw[:9] + bw[10:-3] + bw[-1:]
        for name in ("magi_slices_build", "magi_default_tile_q", "magi_schedule", "magi_qknorm_rope",
                     "magi_ffa_fwd", "magi_ffa_fwd_timed", "magi_ffa_fwd_qknorm", "magi_default_tile_k", "magi_schedule_kv", "magi_ffa_bwd",
                     "magi_ffa_bwd_noalloc",
                     "magi_slices_cross", "magi_slices_ring", "magi_slices_window"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def check(status: int) -> int:
    if status < 0:
        raise MagiError(status, lib().magi_last_error().decode())
    return status


def last_error() -> str:
    return lib().magi_last_error().decode()
