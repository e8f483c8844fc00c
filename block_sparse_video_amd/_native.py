"""ctypes binding of libvsa.so (include/vsa.h).  Argument marshalling only:
every step of the forward pass runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvsa.so")

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every symbol include/vsa.h declares
SIGNATURES = {
    "vsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "vsa_topk_count": (_I32, [_I64, _F32]),
    "vsa_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64, _F32]),
    "vsa_workspace_layout": (ctypes.c_int, [_I32, _I64, _I64, _I64, ctypes.POINTER(_SZ)]),
    "vsa_forward": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P, _P, _SZ, _P]),
    "vsa_pool_pack": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I64, _I64, _P, _SZ, _P]),
    "vsa_select_coarse": (ctypes.c_int, [_I32, _I64, _I64, _I64, _F32, _P, _P, _SZ, _P]),
    "vsa_fine_attention": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P, _P, _SZ, _P]),
    "vsa_project_qkvg": (ctypes.c_int, [_P, _P, _I64, _I32, _I32, _P, _P, _P, _P, _P]),
    "vsa_forward_padded": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64,
                                          _I64, _I64, _I64, _F32, _P, _P, _P, _P, _SZ, _P]),
    "vsa_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P,
                                           _P]),
    "vsa_subblock_whole_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64]),
    "vsa_forward_subblock_whole": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I64, _I64, _F32, _P,
                                                  _P, _P, _SZ, _P]),
    "vsa_subblock_select_whole": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P,
                                                 _SZ, _P]),
    "vsa_subblock_count": (_I32, [_I64, _F32]),
    "vsa_subblock_workspace_bytes": (_SZ, [_I32, _I64, _I64, _I64]),
    "vsa_forward_subblock": (ctypes.c_int, [_P, _P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P, _P,
                                            _SZ, _P]),
    "vsa_subblock_select": (ctypes.c_int, [_P, _P, _I32, _I64, _I64, _I64, _F32, _P, _P, _SZ, _P]),
}

_lib = None


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load the built library.  There is no fallback: a missing library is an error."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              f"or python -m block_sparse_video_amd.build")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().vsa_status_string(status).decode()
