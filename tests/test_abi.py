"""The C-ABI library: loads, exports the declared symbols, validates
arguments and sizes workspaces without touching a GPU (CPU only)."""
import ctypes as C
import os
import re

import pytest

import long_context_decode_fd_amd as fd
from long_context_decode_fd_amd import _abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "fd.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fd_[a-z_0-9]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert "fd_decode_attn" in names and "fd_ffd_sparse_decode" in names
    lib = C.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.SIGNATURES) | {"fd_last_error"}
    assert fd.lib().fd_abi_version() == 1


def test_workspace_sizes():
    # O partials [B,Hq,nc,d] fp32 + (m,l) [B,Hq,nc,2] fp32, each 256-aligned
    n = fd.workspace_bytes("fd_decode_attn", B=8, Hq=32, Hkv=8, L=32768, d=128, chunk=512)
    assert n == 8 * 32 * 64 * 128 * 4 + 8 * 32 * 64 * 2 * 4
    n = fd.workspace_bytes("fd_decode_attn", B=1, Hq=1, Hkv=1, L=1, d=64, chunk=16)
    assert n == 512
    n = fd.workspace_bytes("fd_decode_attn_paged", B=2, Hq=8, Hkv=2, d=128, page=16,
                           max_pages=10, max_seq_len=160, chunk=64)
    assert n == 2 * 8 * 3 * 128 * 4 + 512      # 384 B of (m, l) rounded up to 512


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), _abi.FD_ERR_UNSUPPORTED),
    (dict(Hq=9), _abi.FD_ERR_ARG),             # not a multiple of Hkv
    (dict(Hq=32, Hkv=2), _abi.FD_ERR_UNSUPPORTED),   # group of 16
    (dict(L=0), _abi.FD_ERR_ARG),
    (dict(chunk=24), _abi.FD_ERR_ARG),
    (dict(chunk=0), _abi.FD_ERR_ARG),
    (dict(B=0), _abi.FD_ERR_ARG),
    (dict(scale=-1.0), _abi.FD_ERR_ARG),
    # units (sequence, kv-head, chunk) beyond 32-bit indices, and a length
    # whose chunk count would wrap in 32-bit arithmetic
    (dict(B=4096, Hq=64, Hkv=64, L=2**31 - 1, chunk=65536), _abi.FD_ERR_UNSUPPORTED),
    (dict(B=1, Hq=16, Hkv=16, L=2**31 - 1, chunk=16), _abi.FD_ERR_UNSUPPORTED),
])
def test_validation_errors(kw, code):
    args = dict(B=2, Hq=8, Hkv=2, L=100, d=128, chunk=32)
    args.update(kw)
    with pytest.raises(fd.FdError) as e:
        fd.workspace_bytes("fd_decode_attn", **args)
    assert e.value.code == code


def test_chunk_count_near_int_max():
    # L + chunk - 1 exceeds 32 bits here; the chunk count must not wrap
    L, chunk, B, Hq = 2**31 - 1, 65536, 1, 8
    nc = -(-L // chunk)
    n = fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=8, L=L, d=128, chunk=chunk)
    assert n == B * Hq * nc * 128 * 4 + B * Hq * nc * 2 * 4


def test_unified_and_ffd_validation():
    with pytest.raises(fd.FdError):
        fd.workspace_bytes("fd_decode_attn_unified_max", B=1, Hq=8, Hkv=2, L=64, d=128,
                           chunk=32, phi=float("inf"))
    with pytest.raises(fd.FdError):
        fd.workspace_bytes("fd_decode_attn_unified_max", B=1, Hq=8, Hkv=2, L=64, d=128,
                           chunk=32, margin_hi=100.0)
    with pytest.raises(fd.FdError):
        fd.workspace_bytes("fd_ffd_sparse_decode", B=1, Hq=8, Hkv=2, L=64, d=128, chunk=48)
    with pytest.raises(fd.FdError):
        fd.workspace_bytes("fd_ffd_sparse_decode", B=1, Hq=8, Hkv=2, L=64, d=128, chunk=32,
                           n_sink=0, n_local=0)
    with pytest.raises(fd.FdError):
        fd.workspace_bytes("fd_ffd_sparse_decode", B=1, Hq=8, Hkv=2, L=64, d=128, chunk=32,
                           delta=-1.0)
    assert fd.workspace_bytes("fd_ffd_sparse_decode", B=1, Hq=8, Hkv=2, L=64, d=128,
                              chunk=32) > 0


def test_paged_validation():
    base = dict(B=2, Hq=8, Hkv=2, d=128, page=16, max_pages=4, max_seq_len=64, chunk=32)
    for bad in (dict(page=12), dict(chunk=40), dict(max_seq_len=65), dict(max_pages=0)):
        kw = dict(base); kw.update(bad)
        with pytest.raises(fd.FdError):
            fd.workspace_bytes("fd_decode_attn_paged", **kw)
    assert fd.workspace_bytes("fd_decode_attn_paged", **dict(base, max_seq_len=0)) == 256


def test_null_pointers_rejected_before_launch():
    lib = fd.lib()
    size = C.c_size_t(1 << 20)
    ws = C.c_void_p(256)      # never dereferenced: validation fails first
    rc = lib.fd_decode_attn(1, None, None, None, None, None, 1, 8, 2, 64, 128, 0.1, 32,
                            ws, C.byref(size), None)
    assert rc == _abi.FD_ERR_ARG
    assert b"NULL" in lib.fd_last_error()


def test_workspace_too_small():
    lib = fd.lib()
    size = C.c_size_t(16)
    rc = lib.fd_decode_attn(1, C.c_void_p(256), C.c_void_p(256), C.c_void_p(256),
                            C.c_void_p(256), None, 1, 8, 2, 64, 128, 0.1, 32,
                            C.c_void_p(256), C.byref(size), None)
    assert rc == _abi.FD_ERR_WORKSPACE


def test_append_validation():
    lib = fd.lib()
    p = C.c_void_p(256)        # never dereferenced: validation fails first
    # contiguous: rows t .. t+M-1 must fit in the cache
    for (M, L_cap, d, t, code) in [(2, 10, 128, 9, _abi.FD_ERR_ARG), (1, 10, 128, -1, _abi.FD_ERR_ARG),
                                   (0, 10, 128, 0, _abi.FD_ERR_ARG), (1, 10, 96, 0, _abi.FD_ERR_UNSUPPORTED)]:
        assert lib.fd_kv_append(1, p, p, p, p, 2, 2, M, L_cap, d, t, None) == code
    assert lib.fd_kv_append(1, None, p, p, p, 2, 2, 1, 10, 128, 0, None) == _abi.FD_ERR_ARG
    assert lib.fd_kv_append(1, C.c_void_p(264), p, p, p, 2, 2, 1, 10, 128, 0, None) == _abi.FD_ERR_ARG
    # paged: page size a power of two in [8, 1024]; positive sizes
    for (page, maxp, P, code) in [(12, 4, 8, _abi.FD_ERR_ARG), (16, 0, 8, _abi.FD_ERR_ARG),
                                  (16, 4, 0, _abi.FD_ERR_ARG), (2048, 4, 8, _abi.FD_ERR_ARG)]:
        assert lib.fd_kv_append_paged(1, p, p, p, p, p, p, 2, 2, 1, 128, page, maxp, P, None) == code
    assert lib.fd_kv_append_paged(1, p, p, p, p, None, p, 2, 2, 1, 128, 16, 4, 8, None) == _abi.FD_ERR_ARG
    assert lib.fd_kv_append_paged(7, p, p, p, p, p, p, 2, 2, 1, 128, 16, 4, 8, None) == _abi.FD_ERR_ARG


def test_multi_row_validation_and_workspace():
    base = dict(B=2, M=4, Hq=8, Hkv=2, L=100, d=128, chunk=32)
    # partials of the B*M*Hq*n_chunks = 2*4*8*4 = 256 rows: O and (m, l)
    assert fd.workspace_bytes("fd_decode_attn_multi", **base) == 256 * 128 * 4 + 256 * 2 * 4
    for bad, code in [(dict(M=9), _abi.FD_ERR_UNSUPPORTED),          # G*M = 36 rows
                      (dict(dt=_abi.FD_F32), _abi.FD_ERR_UNSUPPORTED),   # fp32 with M >= 2
                      (dict(M=0), _abi.FD_ERR_ARG), (dict(L=3), _abi.FD_ERR_ARG),
                      (dict(chunk=20), _abi.FD_ERR_ARG)]:
        kw = dict(base); kw.update(bad)
        with pytest.raises(fd.FdError) as e:
            fd.workspace_bytes("fd_decode_attn_multi", **kw)
        assert e.value.code == code, bad
    # one token: the single-query path, any dtype
    assert fd.workspace_bytes("fd_decode_attn_multi", **dict(base, M=1, dt=_abi.FD_F32)) > 0
