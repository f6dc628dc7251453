"""ctypes view of libmars.so (include/mars.h).  Marshalling only: no computation here."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmars.so")

MARS_OK = 0
MARS_EINVAL = -1
MARS_EUNSUPPORTED = -2
MARS_EWORKSPACE = -3
MARS_EHIP = -4
MARS_DTYPE_BF16 = 0
MARS_DTYPE_FP32 = 1
MARS_COMMIT_PER_SAMPLE = 0
MARS_COMMIT_BATCH_MIN = 1

I64x3 = ctypes.c_int64 * 3


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("prompt_len", ctypes.c_int32), ("resp_len", ctypes.c_int32),
        ("block", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("q_strides", I64x3), ("k_strides", I64x3), ("v_strides", I64x3), ("o_strides", I64x3),
    ]


class AttnBwdStrides(ctypes.Structure):
    _fields_ = [("do_strides", I64x3), ("dq_strides", I64x3), ("dk_strides", I64x3), ("dv_strides", I64x3)]


class CeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("prompt_len", ctypes.c_int32), ("resp_len", ctypes.c_int32),
        ("block", ctypes.c_int32), ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("logits_strides", ctypes.c_int64 * 2), ("dlogits_strides", ctypes.c_int64 * 2),
        ("tokens_stride", ctypes.c_int64),
    ]


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32), ("cache_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("scale", ctypes.c_float),
        ("qw_strides", I64x3), ("kw_strides", I64x3), ("vw_strides", I64x3),
        ("kc_strides", I64x3), ("vc_strides", I64x3), ("o_strides", I64x3),
    ]


class AcceptDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("window", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("batch_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64),
        ("tau", ctypes.c_float), ("min_accept", ctypes.c_int32),
    ]


P = ctypes.c_void_p
_SIGNATURES = {
    "mars_abi_version": (ctypes.c_int, []),
    "mars_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "mars_attn_fwd": (ctypes.c_int, [ctypes.POINTER(AttnDesc), P, P, P, P, P, P]),
    "mars_attn_work": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "mars_mask_materialize": (ctypes.c_int, [ctypes.POINTER(AttnDesc), P, P]),
    "mars_tile_map": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.c_int32, ctypes.c_int32, P, P]),
    "mars_attn_tilelog_geometry": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]),
    "mars_attn_fwd_tilelog": (ctypes.c_int, [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P]),
    "mars_attn_bwd_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "mars_attn_bwd_plan": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(ctypes.c_int32)]),
    "mars_attn_bwd": (ctypes.c_int, [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnBwdStrides), P, P, P, P, P, P,
                                     P, P, P, P, ctypes.c_size_t, P]),
    "mars_decode_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(DecodeDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "mars_decode_step": (ctypes.c_int, [ctypes.POINTER(DecodeDesc), P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "mars_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(DecodeDesc), P, P, P, P, P, P, P, P]),
    "mars_decode_scratch_bytes": (ctypes.c_int, [ctypes.POINTER(ctypes.c_size_t)]),
    "mars_kv_commit": (ctypes.c_int, [ctypes.POINTER(DecodeDesc), P, P, P, P, P, P, P, P, ctypes.c_int32, P]),
    "mars_shifted_ce_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(CeDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "mars_shifted_ce": (ctypes.c_int, [ctypes.POINTER(CeDesc), P, P, P, P, P, P, ctypes.c_size_t, P]),
    "mars_accept_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(AcceptDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "mars_accept": (ctypes.c_int, [ctypes.POINTER(AcceptDesc), P, P, P, P, P, ctypes.c_size_t, P]),
    "mars_accept_margin": (ctypes.c_int, [ctypes.POINTER(AcceptDesc), P, P, P, P, P, P, ctypes.c_size_t, P]),
}

_lib = None


def load():
    """Load libmars.so once; raise (never fall back) if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m structured_mask_attention_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGNATURES)
