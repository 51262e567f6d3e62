"""ctypes declarations of the C ABI in include/sla.h (libsla_mi355x.so).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsla_mi355x.so")

SLA_OK, SLA_ERR_NULL, SLA_ERR_INVALID, SLA_ERR_UNSUPPORTED, SLA_ERR_WORKSPACE, SLA_ERR_HIP, \
    SLA_ERR_DEVICE = range(7)
SLA_F32, SLA_BF16 = 0, 1
SLA_OP_FWD, SLA_OP_BWD, SLA_OP_BWD_RECOMPUTE = 0, 1, 2
SLA_SCHED_RECORD_INTS = 12
SLA_BWD_ALL, SLA_BWD_PREPARE, SLA_BWD_DKDV, SLA_BWD_DQ = 0, 1, 2, 3
SLA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024
STU_REUSE_SCHEDULE = 1

# every symbol include/sla.h declares
EXPORTS = (
    "sla_workspace_size", "sla_fwd", "sla_fwd_candidates_workspace_size",
    "sla_fwd_candidates", "sla_bwd", "sla_bwd_noalloc", "sla_bwd_stage", "sla_schedule_capacity", "sla_schedule_tile",
    "sla_schedule", "sla_schedule_host", "sla_ds_blocks_host", "sla_count_pairs_host", "stu_layer_workspace_size", "stu_layer_fwd",
    "stu_layer_bwd_workspace_size", "stu_layer_bwd", "stu_quantize_rows_fp8",
    "stu_layer_fp8_workspace_size", "stu_layer_fwd_fp8", "stu_gather_targets", "stu_truncate", "stu_truncate_bwd", "sla_probe_scratch_size",
    "sla_probe_mfma_peak", "sla_probe_issue_rates", "sla_status_string",
    "sla_last_error",
)


class SLAProblem(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("offsets", ctypes.c_void_p),
        ("num_targets", ctypes.c_void_p),
        ("num_heads", ctypes.c_int32),
        ("d_qk", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("k1", ctypes.c_int32),
        ("k2", ctypes.c_int32),
        ("contextual_len", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("out_f32", ctypes.c_int32),
    ]


class STULayerDesc(ctypes.Structure):
    _fields_ = [("attn", SLAProblem), ("hidden", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("flags", ctypes.c_int32)]


class SLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Load libsla_mi355x.so (once).  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build the HIP library first "
                "(python -m sparse_sequence_attention_amd.build)")
        lib = ctypes.CDLL(path)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        PP = ctypes.POINTER(SLAProblem)
        lib.sla_workspace_size.argtypes = [PP, ctypes.c_int]
        lib.sla_workspace_size.restype = sz
        lib.sla_fwd.argtypes = [PP, P, i64, P, i64, P, i64, P, i64, P, sz, P]
        lib.sla_fwd.restype = ctypes.c_int
        lib.sla_bwd.argtypes = [PP, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P, sz,
                                P]
        lib.sla_bwd.restype = ctypes.c_int
        lib.sla_bwd_noalloc.argtypes = [PP, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P,
                                        i64, P]
        lib.sla_bwd_noalloc.restype = ctypes.c_int
        lib.sla_bwd_stage.argtypes = [PP, ctypes.c_int, P, i64, P, i64, P, i64, P, i64, P, i64, P,
                                      i64, P, i64, P, sz, P]
        lib.sla_bwd_stage.restype = ctypes.c_int
        lib.sla_fwd_candidates_workspace_size.argtypes = [PP, i64]
        lib.sla_fwd_candidates_workspace_size.restype = sz
        lib.sla_fwd_candidates.argtypes = [PP, P, i64, P, i64, P, i64, P, i64, P, i64, P, i64, P,
                                           i64, P, sz, P]
        lib.sla_fwd_candidates.restype = ctypes.c_int
        lib.sla_schedule_capacity.argtypes = [PP, ctypes.c_int]
        lib.sla_schedule_capacity.restype = i64
        lib.sla_schedule_tile.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.sla_schedule_tile.restype = i32
        lib.sla_schedule.argtypes = [PP, ctypes.c_int, P, i64, P, P, sz, P]
        lib.sla_schedule.restype = ctypes.c_int
        lib.sla_schedule_host.argtypes = [PP, ctypes.c_int, P, P, P, i64]
        lib.sla_schedule_host.restype = i64
        lib.sla_ds_blocks_host.argtypes = [PP, P, P, P, i64]
        lib.sla_ds_blocks_host.restype = i64
        lib.sla_count_pairs_host.argtypes = [i32, P, P, i32, i32, i32]
        lib.sla_count_pairs_host.restype = i64
        DBL = ctypes.POINTER(ctypes.c_double)
        lib.sla_probe_scratch_size.argtypes = []
        lib.sla_probe_scratch_size.restype = sz
        lib.sla_probe_mfma_peak.argtypes = [i32, P, sz, DBL, DBL, P]
        lib.sla_probe_mfma_peak.restype = i32
        lib.sla_probe_issue_rates.argtypes = [i32, P, sz, DBL, i32, P]
        lib.sla_probe_issue_rates.restype = i32
        DP = ctypes.POINTER(STULayerDesc)
        lib.stu_layer_workspace_size.argtypes = [DP]
        lib.stu_layer_workspace_size.restype = sz
        lib.stu_layer_fwd.argtypes = [DP, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.stu_layer_fwd.restype = ctypes.c_int
        lib.stu_layer_bwd_workspace_size.argtypes = [DP]
        lib.stu_layer_bwd_workspace_size.restype = sz
        lib.stu_layer_bwd.argtypes = [DP] + [P] * 21 + [sz, P]
        lib.stu_layer_bwd.restype = ctypes.c_int
        lib.stu_quantize_rows_fp8.argtypes = [P, i64, i32, P, P, P]
        lib.stu_quantize_rows_fp8.restype = ctypes.c_int
        lib.stu_layer_fp8_workspace_size.argtypes = [DP]
        lib.stu_layer_fp8_workspace_size.restype = sz
        lib.stu_layer_fwd_fp8.argtypes = [DP] + [P] * 15 + [sz, P]
        lib.stu_layer_fwd_fp8.restype = ctypes.c_int
        lib.stu_gather_targets.argtypes = [i32, i64, P, P, P, i32, i32, P, P, i64, i64, i64, P]
        lib.stu_gather_targets.restype = ctypes.c_int
        lib.stu_truncate_bwd.argtypes = [i32, i64, P, P, i32, i32, P, P, i32, i32, P, P]
        lib.stu_truncate_bwd.restype = ctypes.c_int
        lib.stu_truncate.argtypes = [i32, i64, P, P, i32, i32, P, i32, i32, P, P, P, P, i64, P]
        lib.stu_truncate.restype = ctypes.c_int
        lib.sla_status_string.argtypes = [ctypes.c_int]
        lib.sla_status_string.restype = ctypes.c_char_p
        lib.sla_last_error.argtypes = []
        lib.sla_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def check(status: int) -> None:
    if status != SLA_OK:
        lib = load()
        msg = lib.sla_last_error().decode(errors="replace")
        name = lib.sla_status_string(status).decode()
        raise SLAError(status, f"{name}: {msg}")
