"""ctypes mirror of include/sikv.h (types, constants and function signatures)."""

from __future__ import annotations

import ctypes as C

ABI_VERSION = 7
FLAG_EXACT_SELECT = 1

STATUS = {
    0: "SIKV_OK",
    -1: "SIKV_ERR_INVALID_ARG",
    -2: "SIKV_ERR_UNSUPPORTED",
    -3: "SIKV_ERR_WORKSPACE",
    -4: "SIKV_ERR_HIP",
}


class CacheDesc(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32),
        ("capacity", C.c_int32),
        ("n_tokens", C.c_int32),
        ("n_sink", C.c_int32),
        ("codes", C.c_void_p),
        ("alpha", C.c_void_p),
        ("mu", C.c_void_p),
        ("k_sink", C.c_void_p),
        ("v", C.c_void_p),
        ("v_stride_b", C.c_int64),
        ("v_stride_h", C.c_int64),
        ("v_stride_t", C.c_int64),
        ("codebook", C.c_void_p),
        ("vrec", C.c_void_p),
        ("v_sink", C.c_void_p),
        ("seq_lens", C.c_void_p),
        ("page_table", C.c_void_p),
        ("page_size", C.c_int32),
        ("pages_per_seq", C.c_int32),
        ("n_pages", C.c_int32),
        ("flags", C.c_int32),
        ("timer", C.c_void_p),
    ]


_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64
_SZ = C.c_size_t
_DESC = C.POINTER(CacheDesc)

# name -> (restype, argtypes); every symbol include/sikv.h declares.
SIGNATURES = {
    "sikv_encode": (_I32, [_DESC, _P, _I64, _I64, _I64, _I32, _I32, _I32, _P, _SZ, _P]),
    "sikv_score_topk": (_I32, [_DESC, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "sikv_sparse_attn": (_I32, [_DESC, _P, _I32, _P, _I32, C.c_float, _P, _P, _SZ, _P]),
    "sikv_decode_step": (_I32, [_DESC, _P, _I32, _I32, C.c_float, _P, _P, _P, _SZ, _P]),
    "sikv_append_decode_step": (_I32, [_DESC, _P, _I64, _I64, _P, _I64, _I64, _P, _I32, _I32,
                                       C.c_float, _P, _P, _P, _SZ, _P]),
    "sikv_append_decode_step_static": (_I32, [_DESC, _P, _I64, _I64, _P, _I64, _I64, _P, _I32,
                                              _I32, C.c_float, _P, _P, _P]),
    "sikv_encode_v": (_I32, [_DESC, _P, _I64, _I64, _I64, _I32, _I32, _P]),
    "sikv_workspace_bytes": (_SZ, [_I32, _DESC, _I32, _I32]),
    "sikv_status_str": (C.c_char_p, [_I32]),
    "sikv_abi_version": (_I32, []),
    "sikv_desc_size": (_SZ, []),
    "sikv_dense_attn": (_I32, [_I32, _I32, _I32, _I32, _P, _P, _I64, _I64, _I64, _P, _I64, _I64,
                               _I64, C.c_float, _P, _P, _SZ, _P, _P]),
    "sikv_dense_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "sikv_kmeans_codebook": (_I32, [_DESC, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P]),
    "sikv_dense_scores": (_I32, [_I32, _I32, _I32, _I32, _P, _P, _I64, _I64, _I64, _P, _P, _P]),
    "sikv_stream_copy": (_I32, [_P, _P, _SZ, _P, _P]),
    "sikv_timer_create": (_I32, [C.POINTER(_P)]),
    "sikv_timer_destroy": (_I32, [_P]),
    "sikv_timer_reset": (_I32, [_P]),
    "sikv_timer_read": (_I32, [_P, _I32, C.POINTER(_I64), C.POINTER(C.c_double)]),
    "sikv_timer_count": (_I32, []),
    "sikv_timer_name": (C.c_char_p, [_I32]),
}


def declare(lib: C.CDLL) -> None:
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
