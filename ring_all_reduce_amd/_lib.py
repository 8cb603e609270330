"""Loader of the HIP library librar.so (built in-tree by ring_all_reduce_amd.build).

There is no fallback: if the library has not been built, lib() raises.
"""
from __future__ import annotations

import ctypes
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().parent / "librar.so"
_LIB = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i64p = ctypes.POINTER(ctypes.c_int64)
_ip = ctypes.POINTER(ctypes.c_int)
_int = ctypes.c_int

# name -> (restype, argtypes); mirrors include/rar.h
SIGNATURES = {
    "rar_plan": (_int, [_int, _i64, _int, _int, ctypes.POINTER(_vp)]),
    "rar_plan_destroy": (_int, [_vp]),
    "rar_rank_stride": (_int, [_i64, _int, _i64p]),
    "rar_rank_stride_candidate": (_int, [_i64, _int, _int, _i64p]),
    "rar_rank_stride_tune": (_int, [_int, _i64, _int, _vp, _i64, _int, _vp, _i64p]),
    "rar_rank_stride_tune_stats": (_int, [_int, _i64, _int, _vp, _i64, _int, _vp, _i64p, _ip, _i64p,
                                          ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    "rar_plan_set_algo": (_int, [_vp, _int]),
    "rar_plan_set_grid": (_int, [_vp, _int]),
    "rar_plan_chunk": (_int, [_vp, _int, _i64p, _i64p, _ip]),
    "rar_plan_traffic": (_int, [_vp, _int, _i64p, _i64p]),
    "rar_allreduce_mean": (_int, [_vp, ctypes.POINTER(_vp), _i64, _vp]),
    "rar_allreduce_sgd": (_int, [_vp, ctypes.POINTER(_vp), _vp, ctypes.c_float, _i64, _vp]),
    "rar_allreduce_ring_noalloc": (_int, [_vp, ctypes.POINTER(_vp), _vp, ctypes.c_float, _i64, _vp]),
    "rar_reduce_scatter_sgd_allgather": (_int, [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                                ctypes.c_float, _i64, _vp]),
    "rar_bucket_plan": (_int, [_int, _i64p, _int, _i64, ctypes.POINTER(_vp)]),
    "rar_bucket_destroy": (_int, [_vp]),
    "rar_bucket_count": (_int, [_vp, _ip, _i64p]),
    "rar_bucket_info": (_int, [_vp, _int, _i64p, _i64p, _ip]),
    "rar_bucket_segment": (_int, [_vp, _int, _int, _ip, _i64p, _i64p, _i64p]),
    "rar_bucket_pack": (_int, [_vp, _int, _int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]),
    "rar_bucket_unpack": (_int, [_vp, _int, _int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]),
    "rar_bucket_allreduce_mean": (_int, [_vp, _int, _int, _int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]),
    "rar_bucket_allreduce_arena": (_int, [_vp, _int, _int, _int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp]),
    "rar_strerror": (ctypes.c_char_p, [_int]),
    "rar_version": (_int, []),
}


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ring_all_reduce_amd.build` "
                           "(there is no fallback implementation)")
    L = ctypes.CDLL(str(LIB_PATH))
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _LIB = L
    return L
