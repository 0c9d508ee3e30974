"""ctypes view of the C ABI in include/kda.h and include/kda_layer.h (no computation here).

The shared library is built in-tree by kimi_delta_attention_03_amd.build. If
it is missing, loading raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda_mi355x.so")

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
          4: "KDA_ERR_HIP"}

# every function include/kda.h declares, with (restype, argtypes)
_vp = ctypes.c_void_p


class KdaFwdParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
        ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32), ("g_dtype", ctypes.c_int32), ("beta_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("chunk_size", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32), ("l2norm_eps", ctypes.c_float),
        ("num_seqs", ctypes.c_int32),
    ]


class KdaWorkspaceInfo(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_size_t), ("records_offset", ctypes.c_size_t),
        ("record_bytes", ctypes.c_size_t), ("chunk_slots", ctypes.c_size_t),
        ("off_w", ctypes.c_size_t), ("off_qg", ctypes.c_size_t), ("off_kg", ctypes.c_size_t),
        ("off_aq", ctypes.c_size_t), ("off_u", ctypes.c_size_t), ("off_gamma", ctypes.c_size_t),
        ("elem_bytes", ctypes.c_int32),
        ("off_chunk_table", ctypes.c_size_t), ("off_seq_table", ctypes.c_size_t),
        ("off_order", ctypes.c_size_t),
        ("segments", ctypes.c_int32), ("segment_chunks", ctypes.c_int32),
    ]


class KdaInputReport(ctypes.Structure):
    _fields_ = [("g_min", ctypes.c_float), ("g_max", ctypes.c_float),
                ("beta_min", ctypes.c_float), ("beta_max", ctypes.c_float),
                ("g_nonfinite", ctypes.c_int64), ("beta_nonfinite", ctypes.c_int64),
                ("cu_first_bad", ctypes.c_int64), ("failed", ctypes.c_int32)]


KDA_VALIDATE_SCRATCH_BYTES = 16384
KDA_NOALLOC_SCRATCH_BYTES = 128 << 20


class KdaGateParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("lower_bound", ctypes.c_float),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


GATE_MODES = {None: 0, "log_decay": 0, "softplus": 1, "lower_bound_sigmoid": 2}


class KdaLayerParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64),
        ("M", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
        ("gate_rank", ctypes.c_int32), ("out_gate_rank", ctypes.c_int32), ("conv_size", ctypes.c_int32),
        ("gate_lower_bound", ctypes.c_float), ("norm_eps", ctypes.c_float), ("l2_eps", ctypes.c_float),
    ]


class KdaLayerWorkspaceInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("total_bytes", "off_q", "off_k", "off_v", "off_g_raw", "off_beta",
                                               "off_o")]


LAYER_WEIGHT_NAMES = ["Wqkv", "conv_q", "conv_k", "conv_v", "Wb", "Wad", "Wau", "A_log", "dt_bias",
                      "Wgd", "Wgu", "norm_w", "Wo"]


class KdaLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_WEIGHT_NAMES]


_P = ctypes.POINTER(KdaFwdParams)
_LP = ctypes.POINTER(KdaLayerParams)
SIGNATURES = {
    "kda_chunk_fwd_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "kda_chunk_fwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_chunk_fwd_stage12": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_chunk_fwd_stage34": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_workspace_layout": (ctypes.c_int, [_P, ctypes.POINTER(KdaWorkspaceInfo)]),
    "kda_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_abi_version": (ctypes.c_int32, []),
    "kda_chunk_fwd_gated": (ctypes.c_int, [_P, ctypes.POINTER(KdaGateParams), _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_chunk_affine_summary": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_affine_apply": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp]),
    "kda_decode_step": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_chunk_bwd_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "kda_chunk_bwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_chunk_bwd_stages": (ctypes.c_int, [_P, ctypes.c_int32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "kda_chunk_fwd_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "kda_validate_inputs": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp,
                                           ctypes.POINTER(KdaInputReport)]),
    "kda_layer_fwd_workspace_bytes": (ctypes.c_int, [_LP, ctypes.POINTER(ctypes.c_size_t)]),
    "kda_gemm_bf16_nt": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64, _vp,
                                        ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int32, _vp]),
    "kda_layer_workspace_layout": (ctypes.c_int, [_LP, ctypes.POINTER(KdaLayerWorkspaceInfo)]),
    "kda_layer_fwd": (ctypes.c_int, [_LP, ctypes.POINTER(KdaLayerWeights), _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
}

_lib = None


def load(path: str | None = None):
    """Load the built library once; raise if it is not there."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"KDA HIP library not built: {p} is missing "
                          "(run `python -m kimi_delta_attention_03_amd.build`)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def check(status: int):
    if status != 0:
        msg = load().kda_last_error().decode(errors="replace")
        if status in (1, 2, 3):
            raise KdaValueError(status, msg)
        raise KdaError(status, msg)


class KdaValueError(KdaError, ValueError):
    pass
