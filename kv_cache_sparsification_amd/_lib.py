"""ctypes loader for libkvs.so (built in-tree by kv_cache_sparsification_amd.build).

Importing this module fails loudly when the library is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvs.so")

KVS_OK, KVS_E_INVAL, KVS_E_NOBLOCKS, KVS_E_STATE, KVS_E_HIP = 0, -1, -2, -3, -4
BLOCK_SIZE = 16

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/kvs.h
SIGNATURES = {
    "kvs_last_error": (ctypes.c_char_p, []),
    "kvs_version": (ctypes.c_char_p, []),
    "kvs_prefill_attn_lse": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                      _vp, _vp, _vp, _vp, _vp]),
    "kvs_window_score": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_float, _vp, _vp]),
    "kvs_topk_select": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "kvs_topk_compact": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp,
                                  _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _vp]),
    "kvs_compact_paged": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _c_int, _vp,
                                   _c_int, _vp, _vp]),
    "kvs_paged_decode_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvs_paged_decode": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                  _c_float, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "kvs_copy_blocks": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp]),
    "kvs_paged_decode_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int,
                                          _c_int, _c_float, _vp, _vp, _vp, _vp, _vp]),
    "kvs_slot_init": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "kvs_decode_select_slot": (_c_int, [_vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp, _vp]),
    "kvs_paged_decode_scored_workspace_size": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "kvs_paged_decode_scored": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int,
                                         _c_int, _c_float, _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "kvs_compact_paged_fp8": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp, _vp, _vp,
                                       _c_int, _vp, _c_int, _vp, _vp]),
    "kvs_paged_decode_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                      _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "kvs_paged_decode_scored_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _c_int, _vp, _vp,
                                             _vp, _c_size, _vp]),
    "kvs_paged_decode_scored_select": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int, _c_int, _c_int,
                                                _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int,
                                                _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "kvs_paged_decode_scored_select_fp8": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _vp, _c_int, _vp, _c_int,
                                                    _c_int, _c_int, _c_int, _c_int, _c_float, _vp, _vp, _vp, _vp, _vp,
                                                    _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "kvs_copy_blocks_fp8": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp]),
    "kvs_prefill_attn_lse_chunk": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                            _c_int, _c_float, _vp, _vp, _vp, _vp, _vp]),
    "kvs_window_score_chunk": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_int, _c_float, _vp, _vp]),
    "kvs_gather_paged": (_c_int, [_vp, _vp, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _c_int, _vp, _vp,
                                  _vp]),
    "kvs_probe_stream_read": (_c_int, [_vp, _c_size, _c_int, ctypes.c_uint32, _vp, _vp]),
    "kvs_probe_timestamp": (_c_int, [_vp, _vp]),
    "kvs_alloc_create": (_c_int, [_c_int, _i32p, _c_int, ctypes.POINTER(_vp)]),
    "kvs_alloc_destroy": (None, [_vp]),
    "kvs_alloc_block": (_c_int, [_vp, _i32p]),
    "kvs_alloc_incref": (_c_int, [_vp, ctypes.c_int32]),
    "kvs_alloc_decref": (_c_int, [_vp, ctypes.c_int32]),
    "kvs_alloc_refcount": (_c_int, [_vp, ctypes.c_int32]),
    "kvs_alloc_num_free": (_c_int, [_vp]),
    "kvs_alloc_free_list": (_c_int, [_vp, _i32p, _c_int]),
    "kvs_alloc_cow": (_c_int, [_vp, ctypes.c_int32, _i32p, ctypes.POINTER(_c_int)]),
}


class KvsError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    # Device memory and streams come from torch, so libkvs must run on the very HIP runtime
    # torch loaded: import torch first, and the loader then resolves libkvs's libamdhip64
    # dependency to that already-loaded copy (matched by its soname).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python kv_cache_sparsification_amd/build.py` "
                          "(the HIP library is required; there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    rts = _hip_runtimes_mapped()
    if len(rts) > 1:
        raise ImportError(f"two HIP runtimes are loaded in this process ({rts}); libkvs must share torch's")
    return lib


lib = _load()


def check(code: int) -> int:
    if code < 0:
        raise KvsError(code, lib.kvs_last_error().decode())
    return code
