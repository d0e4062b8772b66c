"""ctypes loader of the HIP library libdit_attn.so (argument marshalling only).

Every entry point of include/dit_attn.h is declared here with its C signature.  The
library must have been built in-tree (partitioned_state_reuse_amd/build.py); there is no
fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdit_attn.so")

c_int, c_float, c_double, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)
P_u8 = ctypes.POINTER(ctypes.c_uint8)
P_f32 = ctypes.POINTER(ctypes.c_float)
P_f64 = ctypes.POINTER(ctypes.c_double)

# name -> (restype, argtypes); mirrors include/dit_attn.h
SIGNATURES = {
    "dit_status_string": (ctypes.c_char_p, [c_int]),
    "dit_attn_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int]),
    "dit_attn_partitioned": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                     P_i32, c_int, P_i32, c_int, P_i32, P_u8, P_u8,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dit_attn_partitioned_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                             P_i32, c_int, P_i32, c_int, P_i32, P_u8, P_u8,
                                             c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                             c_void_p, c_void_p, c_void_p]),
    "dit_partition_attention": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                        P_i32, c_int, P_i32, c_int, P_i32, P_u8, P_u8,
                                        c_void_p, c_void_p, c_float, c_void_p, c_size_t, c_void_p]),
    "dit_partition_attention_premerge": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                                 P_i32, c_int, P_i32, c_int, P_i32, P_u8, P_u8,
                                                 c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                                 c_void_p, c_size_t, c_void_p]),
    "dit_partition_attention_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                            P_i32, c_int, P_i32, c_int, P_i32, P_u8, P_u8,
                                            c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_size_t, c_void_p]),
    "dit_state_merge_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                    c_void_p, c_void_p, P_i32, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dit_state_merge": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, P_i32, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dit_state_merge_masked": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, P_i32, c_int, P_u8,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dit_state_compose": (c_int, [c_void_p, c_void_p, c_int, P_i32, c_int, c_int, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_void_p]),
    "dit_importance": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, P_i32, c_int,
                               c_void_p, c_void_p]),
    "dit_local_change_finalize": (c_int, [c_void_p, c_size_t, c_int, c_int, c_int, c_int, P_i32, c_int,
                                          c_void_p, c_void_p]),
    "dit_planner_create": (c_int, [c_int, c_int, P_i32, c_int, P_i32, c_int, c_int, c_int,
                                   ctypes.POINTER(c_void_p)]),
    "dit_planner_next": (c_int, [c_void_p, c_int, P_u8, P_i32]),
    "dit_planner_observe": (c_int, [c_void_p, c_int, P_f32, P_f32]),
    "dit_planner_scores": (c_int, [c_void_p, c_int, P_f64]),
    "dit_planner_destroy": (None, [c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with partitioned_state_reuse_amd/build.py "
                               f"(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
