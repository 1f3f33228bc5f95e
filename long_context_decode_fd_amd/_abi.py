"""ctypes declarations of the C ABI in include/fd.h.

Loading fails loudly when the shared library has not been built: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

# FD_AMD_LIB selects another build of the same ABI (the host-sanitizer
# build of the CPU checks); by default the in-tree library.
LIB_PATH = os.environ.get("FD_AMD_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfd_amd.so")

FD_F32, FD_BF16 = 0, 1
FD_OK, FD_ERR_ARG, FD_ERR_UNSUPPORTED, FD_ERR_WORKSPACE, FD_ERR_HIP = range(5)
FD_NOALLOC_BYTES = 32 << 20   # the library-owned partials buffer of fd_decode_attn_noalloc
ERROR_NAMES = {FD_ERR_ARG: "FD_ERR_ARG", FD_ERR_UNSUPPORTED: "FD_ERR_UNSUPPORTED",
               FD_ERR_WORKSPACE: "FD_ERR_WORKSPACE", FD_ERR_HIP: "FD_ERR_HIP"}

_vp, _i, _f, _szp = C.c_void_p, C.c_int, C.c_float, C.POINTER(C.c_size_t)

# name -> argument types (all return int except fd_last_error)
SIGNATURES = {
    "fd_abi_version": [],
    "fd_decode_attn": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                       _vp, _szp, _vp],
    "fd_decode_attn_noalloc": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp],
    "fd_decode_attn_partials": [_i, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _szp,
                                _vp],
    "fd_merge_partials": [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp],
    "fd_decode_attn_paged": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                             _i, _i, _i, _i, _f, _i, _vp, _szp, _vp],
    "fd_decode_attn_unified_max": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                   _f, _i, _f, _f, _f, _vp, _vp, _szp, _vp],
    "fd_decode_attn_multi": [_i, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                             _vp, _szp, _vp],
    "fd_decode_attn_multi_paged": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                   _i, _i, _i, _i, _i, _f, _i, _vp, _szp, _vp],
    "fd_kv_append": [_i, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp],
    "fd_kv_append_paged": [_i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                           _vp],
    "fd_ffd_pack": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp],
    "fd_ffd_sparse_decode": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                             _i, _f, _f, _i, _i, _i, _vp, _vp, _vp, _szp, _vp],
}

_lib = None


class FdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def load(path: str = LIB_PATH):
    """Load (once) and return the library with typed entry points."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m long_context_decode_fd_amd.build` "
            "(there is no fallback implementation)")
    lib = C.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_int
    lib.fd_last_error.argtypes = []
    lib.fd_last_error.restype = C.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def check(code: int, lib=None):
    if code != FD_OK:
        lib = lib or load()
        raise FdError(code, lib.fd_last_error().decode())
