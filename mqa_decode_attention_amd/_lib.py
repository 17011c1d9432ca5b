"""ctypes loader for libkvc.so (the HIP kernels and their C ABI, include/kvc.h).

The library is built in-tree by ``python -m mqa_decode_attention_amd.build``.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvc.so")

c_int, c_longlong, c_size_t, c_float, c_void_p, c_char_p = (ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t,
                                                             ctypes.c_float, ctypes.c_void_p, ctypes.c_char_p)

# name -> (restype, argtypes); mirrors include/kvc.h
SIGNATURES = {
    "kvc_abi_version": (c_int, []),
    "kvc_status_string": (c_char_p, [c_int]),
    "kvc_last_error": (c_char_p, []),
    "kvc_profile_next_decode": (None, [c_void_p, c_void_p]),
    "kvc_hbm_read_probe": (c_int, [c_void_p, c_size_t, c_void_p, c_int, c_int, c_void_p]),
    "kvc_append": (c_int, [c_int, c_int, c_int, c_int, c_int,
                           c_void_p, c_void_p, c_int,
                           c_void_p, c_int, c_int, c_int, c_void_p,
                           c_void_p, c_void_p, c_void_p,
                           c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "kvc_decode_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_longlong, c_int]),
    "kvc_workspace_zeroed_bytes": (c_size_t, []),
    "kvc_decode_merge_launch": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_longlong, c_int]),
    "kvc_decode_balanced": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_longlong, c_int]),
    "kvc_decode_compact": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_longlong, c_int]),
    "kvc_decode_split_tokens": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_longlong, c_int]),
    "kvc_decode_attn": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_void_p, c_int,
                                c_void_p, c_int, c_float, c_void_p,
                                c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_attn_paged": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p,
                                      c_int, c_int, c_void_p, c_int, c_void_p,
                                      c_int, c_float, c_void_p, c_int,
                                      c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                c_void_p, c_int, c_int, c_int, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p,
                                c_int, c_int, c_int, c_float, c_void_p,
                                c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step_noalloc": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                        c_void_p, c_int, c_int, c_int, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_int, c_int, c_int, c_float, c_void_p,
                                        c_int, c_void_p]),
    "kvc_decode_step_noalloc_max_bytes": (c_size_t, []),
    "kvc_append_ring": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                c_void_p, c_void_p, c_int, c_void_p,
                                c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "kvc_window_span": (c_int, [c_int, c_int, c_int, c_int]),
    "kvc_decode_attn_window": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                       c_void_p, c_void_p, c_void_p, c_int,
                                       c_void_p, c_int, c_int, c_int, c_void_p,
                                       c_int, c_int, c_int, c_float, c_void_p,
                                       c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step_window": (c_int, [c_int, c_int, c_int, c_int, c_int,
                                       c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                       c_void_p, c_int, c_int, c_int, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int, c_int, c_int, c_int, c_int, c_float, c_void_p,
                                       c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_append_multi": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                                 c_void_p, c_void_p, c_int,
                                 c_void_p, c_int, c_int, c_int, c_void_p,
                                 c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "kvc_decode_multi_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                                    c_longlong, c_int]),
    "kvc_decode_multi_split_tokens": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                              c_longlong, c_int]),
    "kvc_decode_attn_multi": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                                      c_void_p, c_void_p, c_void_p, c_int,
                                      c_void_p, c_int, c_int, c_int, c_void_p,
                                      c_int, c_int, c_float, c_void_p,
                                      c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_append_u8": (c_int, [c_int, c_int, c_int, c_int, c_int,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                              c_void_p, c_int, c_int, c_int, c_void_p,
                              c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "kvc_decode_attn_u8": (c_int, [c_int, c_int, c_int, c_int, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                   c_void_p, c_int, c_float, c_void_p,
                                   c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_attn_paged_u8": (c_int, [c_int, c_int, c_int, c_int, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                         c_int, c_void_p, c_int,
                                         c_void_p, c_int, c_float, c_void_p,
                                         c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step_u8": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_float,
                                   c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_append_fp8": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                               c_void_p, c_int, c_int, c_int, c_void_p,
                               c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "kvc_decode_attn_fp8": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                    c_void_p, c_int, c_float, c_void_p,
                                    c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_attn_paged_fp8": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                          c_int, c_void_p, c_int,
                                          c_void_p, c_int, c_float, c_void_p,
                                          c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step_fp8": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_float,
                                    c_void_p, c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_append_mla": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "kvc_decode_mla_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
    "kvc_decode_mla_split_tokens": (c_int, [c_int, c_int, c_int, c_int, c_int]),
    "kvc_decode_attn_mla": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p,
                                    c_void_p, c_int, c_void_p, c_int,
                                    c_void_p, c_void_p, c_void_p, c_float, c_void_p,
                                    c_int, c_void_p, c_size_t, c_void_p]),
    "kvc_decode_step_mla": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_void_p,
                                    c_int, c_void_p, c_void_p,
                                    c_void_p, c_int, c_void_p, c_void_p,
                                    c_void_p, c_float, c_void_p, c_int, c_void_p,
                                    c_size_t, c_void_p]),
}

ABI_VERSION = 14

_lib = None


def load() -> ctypes.CDLL:
    """Load libkvc.so once and declare every exported function's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m mqa_decode_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.kvc_abi_version() != ABI_VERSION:
        raise ImportError(f"libkvc ABI {lib.kvc_abi_version()} != expected {ABI_VERSION}; rebuild it")
    _lib = lib
    return lib
