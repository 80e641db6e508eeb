"""ctypes view of include/kda.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libkda.so")

KDA_OK = 0
STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_NULL_POINTER", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_CHUNK_SIZE",
    4: "KDA_ERR_HEAD_DIM", 5: "KDA_ERR_UNSUPPORTED", 6: "KDA_ERR_GVA", 7: "KDA_ERR_MISSING_A_LOG",
    8: "KDA_ERR_LOWER_BOUND", 9: "KDA_ERR_NEG_EIGVAL", 10: "KDA_ERR_VARLEN", 11: "KDA_ERR_DTYPE",
    12: "KDA_ERR_WORKSPACE", 13: "KDA_ERR_HIP",
}
STATUS = {v: k for k, v in STATUS_NAMES.items()}
KDA_ERR_HIP = STATUS["KDA_ERR_HIP"]

DTYPE_FP32, DTYPE_BF16 = 0, 1

GATE_IN_KERNEL = 1 << 0
SAFE_GATE = 1 << 1
HAS_LOWER_BOUND = 1 << 2
QK_L2NORM = 1 << 3
BETA_SIGMOID = 1 << 4
ALLOW_NEG_EIGVAL = 1 << 5
OUTPUT_FINAL_STATE = 1 << 6
TRANSPOSE_STATE = 1 << 7

# every function include/kda.h declares
EXPORTS = (
    "kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd",
    "kda_gate_chunk_cumsum_workspace_size", "kda_gate_chunk_cumsum", "kda_chunk_fwd_stage_count",
    "kda_chunk_fwd_stage_name", "kda_chunk_fwd_profiled", "kda_fused_recurrent_fwd", "kda_chunk_fwd_states",
    "kda_chunk_bwd_workspace_size", "kda_chunk_bwd", "kda_chunk_fwd_noalloc",
    "kda_chunk_bwd_tokenwise_workspace_size", "kda_chunk_bwd_tokenwise", "kda_chunk_fwd_save",
    "kda_chunk_bwd_saved",
)
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class KdaFwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("HV", ctypes.c_int32),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32), ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int64)),
        ("qkv_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("lower_bound", ctypes.c_float), ("flags", ctypes.c_uint32),
    ]


_vp = ctypes.c_void_p
_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libkda.so.  There is no fallback: a missing library is an error."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m gated_delta_rule_log2_amd.build` "
            "(or __graft_entry__.build()); the KDA path has no CPU fallback")
    # torch first: its HIP runtime (SONAME libamdhip64.so.7) then satisfies this
    # library's dependency, so one process holds a single HIP runtime whose
    # streams and device pointers both sides share.
    import torch  # noqa: F401

    lib = ctypes.CDLL(path)
    lib.kda_abi_version.restype = ctypes.c_int
    lib.kda_abi_version.argtypes = []
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    dp = ctypes.POINTER(KdaFwdDesc)
    szp = ctypes.POINTER(ctypes.c_size_t)
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace_size.argtypes = [dp, szp]
    lib.kda_gate_chunk_cumsum_workspace_size.restype = ctypes.c_int
    lib.kda_gate_chunk_cumsum_workspace_size.argtypes = [dp, szp]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  ctypes.c_size_t, _vp]
    lib.kda_chunk_fwd_states.restype = ctypes.c_int
    lib.kda_chunk_fwd_states.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]
    lib.kda_chunk_fwd_profiled.restype = ctypes.c_int
    lib.kda_chunk_fwd_profiled.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp, _vp]
    lib.kda_chunk_fwd_stage_count.restype = ctypes.c_int
    lib.kda_fused_recurrent_fwd.restype = ctypes.c_int
    lib.kda_fused_recurrent_fwd.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.kda_chunk_fwd_stage_count.argtypes = []
    lib.kda_chunk_fwd_stage_name.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_stage_name.argtypes = [ctypes.c_int]
    lib.kda_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_size.argtypes = [dp, szp]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = [dp] + [_vp] * 20 + [ctypes.c_size_t, _vp]
    lib.kda_chunk_bwd_tokenwise_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_bwd_tokenwise_workspace_size.argtypes = [dp, szp]
    lib.kda_chunk_bwd_tokenwise.restype = ctypes.c_int
    lib.kda_chunk_bwd_tokenwise.argtypes = [dp] + [_vp] * 20 + [ctypes.c_size_t, _vp]
    lib.kda_chunk_fwd_save.restype = ctypes.c_int
    lib.kda_chunk_fwd_save.argtypes = [dp] + [_vp] * 12 + [ctypes.c_size_t, _vp]
    lib.kda_chunk_bwd_saved.restype = ctypes.c_int
    lib.kda_chunk_bwd_saved.argtypes = [dp] + [_vp] * 20 + [ctypes.c_size_t, _vp]
    lib.kda_gate_chunk_cumsum.restype = ctypes.c_int
    lib.kda_gate_chunk_cumsum.argtypes = [dp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    if path == LIBRARY:
        _lib = lib
    return lib
