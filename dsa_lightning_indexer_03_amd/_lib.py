"""ctypes loader of libdsaidx.so: one Python function per C entry point,
argument types declared, nothing else.  Raises if the library is missing --
there is no fallback."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsaidx.so")

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size_t = ctypes.c_size_t
_c_int64 = ctypes.c_int64

# (name, restype, argtypes) for every symbol declared in include/dsaidx.h
SIGNATURES = {
    "indexer_prefill": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p,
                                 _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "indexer_prefill_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "indexer_prefill_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_void_p,
                                         _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "indexer_prefill_noalloc_scratch_bytes": (_c_size_t, []),
    "indexer_decode_paged": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                      _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "indexer_decode_paged_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "topk_select": (_c_int, [_c_void_p, _c_int, _c_int, _c_int64, _c_void_p, _c_int, _c_void_p, _c_void_p,
                             _c_void_p, _c_size_t, _c_void_p]),
    "topk_select_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int]),
    "indexer_kcache_append": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                       _c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p]),
    "indexer_prefill_chunk_paged": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_void_p, _c_void_p, _c_void_p,
                                             _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "indexer_prefill_chunk_paged_workspace_bytes": (_c_size_t, [_c_int, _c_int, _c_int, _c_int]),
    "indexer_topk_gather": (_c_int, [_c_void_p, _c_int, _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_int,
                                     _c_int, _c_void_p, _c_void_p]),
    "indexer_topk_gather_layers": (_c_int, [ctypes.POINTER(_c_void_p), ctypes.POINTER(_c_void_p), _c_int, _c_int,
                                            _c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_int, _c_int,
                                            _c_void_p]),
    "dsaidx_probe_mfma": (_c_int, [_c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "dsaidx_probe_page_read": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_int, _c_int, _c_void_p, _c_void_p]),
    "dsaidx_status_string": (ctypes.c_char_p, [_c_int]),
    "dsaidx_last_error": (ctypes.c_char_p, []),
    "dsaidx_version": (_c_int, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the library once and declares every signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m dsa_lightning_indexer_03_amd.build` "
                          "(or __graft_entry__.build()); there is no non-HIP fallback")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class DsaidxError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.dsaidx_status_string(status).decode()
        detail = lib.dsaidx_last_error().decode()
        super().__init__(f"{where}: status {status} ({msg}): {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != 0:
        raise DsaidxError(status, where)
