"""ctypes view of libcpla.so (argument marshalling only).

The library must have been built in-tree (``__graft_entry__.build()`` or
``python -m context_state_passing_amd.build``); importing a function from here
without it raises immediately -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpla.so")

F32, BF16 = 0, 1
DECAY_NONE, DECAY_SCALAR, DECAY_DIAG, DECAY_DELTA = 0, 1, 2, 3
STATUS = {0: "OK", 1: "INVALID", 2: "SHAPE", 3: "DTYPE", 4: "ALIGN", 5: "UNSUPPORTED", 6: "METADATA", 7: "HIP"}

# every function the header include/cpla.h declares
EXPORTS = [
    "cpla_summary_width", "cpla_chunk_states_bytes", "cp_forward_prepare", "cp_forward_apply",
    "cp_backward_prepare", "cp_backward_apply", "build_packed_sequence_cp_metadata",
    "cpla_packed_rank_slices", "cpla_seq_idx_from_cu_seqlens", "cpla_last_error", "cpla_abi_version",
    "cpla_ssd_inputs", "cpla_ssd_input_grads", "cp_forward_prepare_weighted", "cp_forward_apply_weighted",
    "cp_backward_apply_weighted", "cpla_delta_workspace_bytes", "cp_forward_prepare_delta",
    "cp_forward_apply_delta", "cp_backward_prepare_delta", "cp_backward_apply_delta",
    "cpla_set_apply_parts", "cp_forward_apply_noalloc", "cpla_noalloc_scratch_bytes",
    "cpla_check_decay_range",
]


class CplaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"cpla {STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("num_shards", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("rank_begin", ctypes.c_int32), ("rank_end", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("decay", ctypes.c_int32), ("qk_heads", ctypes.c_int32)]


class SsdProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("G", ctypes.c_int64),
                ("N", ctypes.c_int64), ("P", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class Packed(ctypes.Structure):
    _fields_ = [("seq_idx", ctypes.c_void_p), ("preceding_rank_start", ctypes.c_void_p),
                ("following_rank_stop", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, V, I32, I64 = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        PK = ctypes.POINTER(Packed)
        pi32 = ctypes.POINTER(ctypes.c_int32)
        L.cpla_summary_width.argtypes = [P]
        L.cpla_summary_width.restype = I64
        L.cpla_chunk_states_bytes.argtypes = [P]
        L.cpla_chunk_states_bytes.restype = I64
        L.cp_forward_prepare.argtypes = [P, PK, V, V, V, V, V]
        L.cp_forward_apply.argtypes = [P, PK, V, V, V, V, V, V, V, V, V, V, V]
        L.cp_backward_prepare.argtypes = [P, PK, V, V, V, V, V]
        L.cp_backward_apply.argtypes = [P, PK, V, V, V, V, V, V, V, V, V, V, V, V, V, V, V]
        for fn in ["cp_forward_prepare", "cp_forward_apply", "cp_backward_prepare", "cp_backward_apply"]:
            getattr(L, fn).restype = ctypes.c_int
        L.build_packed_sequence_cp_metadata.argtypes = [pi32, I64, I32, I32, pi32, pi32, pi32, pi32, pi32]
        L.build_packed_sequence_cp_metadata.restype = ctypes.c_int
        L.cpla_packed_rank_slices.argtypes = [pi32, I64, I32, pi32, pi32]
        L.cpla_packed_rank_slices.restype = ctypes.c_int
        L.cpla_seq_idx_from_cu_seqlens.argtypes = [pi32, I32, I64, pi32]
        L.cpla_seq_idx_from_cu_seqlens.restype = ctypes.c_int
        SP = ctypes.POINTER(SsdProblem)
        L.cpla_ssd_inputs.argtypes = [SP, V, V, V, V, V, V, V, V]
        L.cpla_ssd_inputs.restype = ctypes.c_int
        L.cpla_ssd_input_grads.argtypes = [SP, V, V, V, V, V, V, V, V, V, V, V, V, V]
        L.cpla_ssd_input_grads.restype = ctypes.c_int
        L.cp_forward_prepare_weighted.argtypes = [P, PK, V, V, V, V, V, V]
        L.cp_forward_apply_weighted.argtypes = [P, PK, V, V, V, V, V, V, V, V, V, V, V, V]
        L.cp_backward_apply_weighted.argtypes = [P, PK, V, V, V, V, V, V, V, V, V, V, V, V, V, V, V, V, I32, V]
        for fn in ["cp_forward_prepare_weighted", "cp_forward_apply_weighted", "cp_backward_apply_weighted"]:
            getattr(L, fn).restype = ctypes.c_int
        L.cpla_delta_workspace_bytes.argtypes = [P]
        L.cpla_delta_workspace_bytes.restype = ctypes.c_int64
        L.cp_forward_prepare_delta.argtypes = [P, PK] + [V] * 7
        L.cp_forward_apply_delta.argtypes = [P, PK] + [V] * 12
        L.cp_backward_prepare_delta.argtypes = [P, PK] + [V] * 9
        L.cp_backward_apply_delta.argtypes = [P, PK] + [V] * 17
        for fn in ["cp_forward_prepare_delta", "cp_forward_apply_delta", "cp_backward_prepare_delta",
                   "cp_backward_apply_delta"]:
            getattr(L, fn).restype = ctypes.c_int
        L.cpla_last_error.restype = ctypes.c_char_p
        L.cpla_abi_version.restype = ctypes.c_int
        L.cp_forward_apply_noalloc.argtypes = [P, PK, V, V, V, V, V, V, V, V, V, V]
        L.cp_forward_apply_noalloc.restype = ctypes.c_int
        L.cpla_noalloc_scratch_bytes.argtypes = []
        L.cpla_noalloc_scratch_bytes.restype = ctypes.c_int64
        L.cpla_check_decay_range.argtypes = [P, V, V, V]
        L.cpla_check_decay_range.restype = ctypes.c_int
        L.cpla_set_apply_parts.argtypes = [ctypes.c_int]
        L.cpla_set_apply_parts.restype = ctypes.c_int
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        msg = lib().cpla_last_error()
        raise CplaError(status, msg.decode() if msg else "")
