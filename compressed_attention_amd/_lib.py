"""ctypes loader for libhattn.so (the HIP library).  No fallback: if the
library is missing the first call raises, naming the build step."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhattn.so")
ABI_VERSION = 3  # hattn_abi_version() of the library this binding matches

_i32, _i64, _f32, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
_psz = ctypes.POINTER(ctypes.c_size_t)

# name -> argument types, in the order of include/hattn.h
SIGNATURES = {
    "hattn_compress": [_i32, _p, _i64, _i64, _i32, _p, _p, _i32, _i32, _i64, _i64, _p, _p],
    "hattn_compress_with_index": [_i32, _p, _p, _i64, _i64, _i32, _i32, _p, _p, _i32, _i32, _i64, _i64, _p, _p, _p],
    "hattn_compress_channel_logits": [_i32, _p, _i64, _i64, _i32, _p, _p, _i32, _i32, _i64, _i64, _p, _p],
    "hattn_visible_count": [_p, _i64, _i32, _i32, _i64, _p, _p],
    "hattn_index_topk": [_i32, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _i32, _p, _p, _p, _psz, _p],
    "hattn_hisa_pool": [_i32, _p, _i64, _i64, _i32, _i32, _i64, _i64, _p, _p],
    "hattn_hisa_topk": [_i32, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i32, _i32, _i32, _p, _p, _p, _psz,
                        _p],
    "hattn_block_sparse_topk": [_i32, _p, _p, _p, _p, _i64, _i64, _i32, _i32, _i64, _p, _i32, _i32, _p, _p, _p, _psz,
                               _p],
    "hattn_sparse_attn": [_i32, _p, _p, _i64, _p, _i32, _p, _i64, _i64, _p, _i32, _f32, _i64, _i64, _i32, _i32, _p,
                          _p, _p, _psz, _p],
    "hattn_sparse_attn_noalloc": [_i32, _p, _p, _i64, _p, _i32, _p, _i64, _i64, _p, _i32, _f32, _i64, _i64, _i32, _i32,
                                  _p, _p, _p],
    "hattn_dense_compressed_attn": [_i32, _p, _p, _i64, _p, _p, _i64, _i64, _p, _i32, _f32, _i64, _i64, _i32, _i32, _p,
                                    _p, _p, _psz, _p],
    "hattn_decode_append": [_i32, _p, _i64, _i64, _i64, _i32, _p, _p, _i32, _i32, _p, _p, _p, _p, _i32, _i32, _p, _p],
    "hattn_decode_desc_size": [],
    "hattn_decode_plan_ws_bytes": [_p, _psz],
    "hattn_decode_plan_create": [_p, ctypes.POINTER(_p)],
    "hattn_decode_plan_run": [_p, _p],
    "hattn_decode_plan_run_graph": [_p, _p],
    "hattn_decode_plan_destroy": [_p],
    "hattn_timer_enable": [_i32],
    "hattn_timer_collect": [],
    "hattn_timer_query": [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
    "hattn_timer_names": [ctypes.c_char_p, _i64],
    "hattn_status_string": [ctypes.c_int],
    "hattn_last_error": [],
    "hattn_abi_version": [],
}



class DecodeDesc(ctypes.Structure):
    """Mirror of hattn_decode_desc (include/hattn.h), field for field."""
    _fields_ = [
        ("dtype", _i32), ("h", _i32), ("d", _i32), ("window", _i32),
        ("bt", _i64), ("L", _i64), ("raw_rows", _i64),
        ("scale", _f32),
        ("h_i", _i32), ("d_i", _i32), ("B", _i32), ("m", _i32), ("k", _i32),
        ("csa_w", _i32), ("csa_stride", _i32), ("hca_w", _i32), ("hca_stride", _i32),
        ("q_pos", _p),
        ("csa_raw_kv", _p), ("csa_logits", _p), ("csa_pos_bias", _p), ("csa_ckv", _p),
        ("k_i", _p), ("reps", _p), ("q_i", _p), ("w_i", _p),
        ("csa_q", _p), ("csa_out", _p), ("csa_lse", _p), ("csa_idx", _p),
        ("hca_raw_kv", _p), ("hca_logits", _p), ("hca_pos_bias", _p), ("hca_ckv", _p),
        ("hca_q", _p), ("hca_out", _p), ("hca_lse", _p),
        ("ws", _p), ("ws_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run __graft_entry__.build() (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.hattn_status_string.restype = ctypes.c_char_p
        L.hattn_last_error.restype = ctypes.c_char_p
        L.hattn_decode_desc_size.restype = ctypes.c_int64
        if L.hattn_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libhattn.so has ABI {L.hattn_abi_version()}, the binding expects {ABI_VERSION}; "
                               "rebuild it with __graft_entry__.build()")
        if L.hattn_decode_desc_size() != ctypes.sizeof(DecodeDesc):
            raise RuntimeError("hattn_decode_desc layout differs between the library and the binding")
        _lib = L
    return _lib


class HattnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.hattn_last_error().decode(errors="replace")
        super().__init__(f"{fn}: {L.hattn_status_string(status).decode()} ({msg})")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise HattnError(fn, status)
