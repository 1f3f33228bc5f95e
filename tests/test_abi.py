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


# The exported C ABI, argument by argument (type, name), as include/fd.h
# declares it.  A change to any signature must change this table, the ctypes
# declarations in _abi.py and fd_abi_version together.
EXPECTED_PROTOTYPES = {
    "fd_last_error": ("const char*", []),
    "fd_abi_version": ("int", []),
    "fd_decode_attn": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k", "const void* v", "float* out",
        "float* lse", "int B", "int Hq", "int Hkv", "int L", "int d", "float scale", "int chunk",
        "void* ws", "size_t* ws_bytes", "void* stream"]),
    "fd_decode_attn_noalloc": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k", "const void* v", "float* out",
        "float* lse", "int B", "int Hq", "int Hkv", "int L", "int d", "float scale", "int chunk",
        "void* stream"]),
    "fd_decode_attn_partials": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k", "const void* v", "int B", "int Hq",
        "int Hkv", "int L", "int d", "float scale", "int chunk", "void* ws", "size_t* ws_bytes",
        "void* stream"]),
    "fd_merge_partials": ("int", [
        "const float* o_part", "const float* ml_part", "float* out", "float* lse", "int B",
        "int Hq", "int n_chunks", "int d", "void* stream"]),
    "fd_decode_attn_paged": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens", "float* out", "float* lse",
        "int B", "int Hq", "int Hkv", "int d", "int page_size", "int max_pages_per_seq",
        "int num_pages", "int max_seq_len", "float scale", "int chunk", "void* ws",
        "size_t* ws_bytes", "void* stream"]),
    "fd_decode_attn_unified_max": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k", "const void* v", "float* out",
        "float* lse", "int B", "int Hq", "int Hkv", "int L", "int d", "float scale", "int chunk",
        "float phi", "float margin_hi", "float margin_lo", "uint8_t* chunk_flags", "void* ws",
        "size_t* ws_bytes", "void* stream"]),
    "fd_decode_attn_multi": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k", "const void* v", "float* out",
        "float* lse", "int B", "int M", "int Hq", "int Hkv", "int L", "int d", "float scale",
        "int chunk", "void* ws", "size_t* ws_bytes", "void* stream"]),
    "fd_decode_attn_multi_paged": ("int", [
        "fd_dtype_t dt", "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens", "float* out", "float* lse",
        "int B", "int M", "int Hq", "int Hkv", "int d", "int page_size", "int max_pages_per_seq",
        "int num_pages", "int max_seq_len", "float scale", "int chunk", "void* ws",
        "size_t* ws_bytes", "void* stream"]),
    "fd_kv_append": ("int", [
        "fd_dtype_t dt", "const void* k_new", "const void* v_new", "void* k_cache",
        "void* v_cache", "int B", "int Hkv", "int M", "int L_cap", "int d", "int t",
        "void* stream"]),
    "fd_kv_append_paged": ("int", [
        "fd_dtype_t dt", "const void* k_new", "const void* v_new", "void* k_pool",
        "void* v_pool", "const int32_t* block_table", "const int32_t* pos", "int B", "int Hkv",
        "int M", "int d", "int page_size", "int max_pages_per_seq", "int num_pages",
        "void* stream"]),
    "fd_ffd_pack": ("int", [
        "const void* k", "uint32_t* codes", "uint16_t* zs", "int8_t* res", "uint16_t* rs",
        "int B", "int Hkv", "int L_cap", "int d", "int t_begin", "int t_end", "void* stream"]),
    "fd_ffd_sparse_decode": ("int", [
        "const void* q", "const uint32_t* codes", "const uint16_t* zs", "const int8_t* res",
        "const uint16_t* rs", "const void* v", "float* out", "float* lse", "int B", "int Hq",
        "int Hkv", "int L", "int d", "float scale", "float delta", "int n_sink", "int n_local",
        "int chunk", "uint32_t* cand_mask", "float* pseudo_max", "void* ws", "size_t* ws_bytes",
        "void* stream"]),
}


def _prototypes():
    """(return type, [argument declarations]) of every function in fd.h."""
    txt = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    found = {}
    for m in re.finditer(r"(int|const char\*)\s+(fd_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", txt):
        args = [" ".join(a.split()) for a in m.group(3).split(",")]
        found[m.group(2)] = (m.group(1), [] if args == ["void"] else args)
    return found


def _ctypes_kind(decl):
    ctype = decl.rsplit(" ", 1)[0]
    if ctype == "size_t*":
        return "size_t*"
    if ctype.endswith("*"):
        return "pointer"
    return {"int": "int", "fd_dtype_t": "int", "float": "float"}[ctype]


def test_exported_argument_lists_are_pinned():
    """The header's prototypes equal the pinned table, and the ctypes
    declarations the binding calls through agree with them argument by
    argument (pointer / size_t* / int / float)."""
    assert _prototypes() == EXPECTED_PROTOTYPES
    kinds = {C.c_void_p: "pointer", C.c_int: "int", C.c_float: "float",
             C.POINTER(C.c_size_t): "size_t*"}
    for name, (ret, args) in EXPECTED_PROTOTYPES.items():
        if name == "fd_last_error":
            continue
        assert ret == "int", name
        assert [kinds[t] for t in _abi.SIGNATURES[name]] == [_ctypes_kind(a) for a in args], name


def test_workspace_sizes():
    # O partials [B,Hq,nc,d] fp32 + (m,l) [B,Hq,nc,2] fp32, each 256-aligned
    n = fd.workspace_bytes("fd_decode_attn", B=8, Hq=32, Hkv=8, L=32768, d=128, chunk=512)
    assert n == 8 * 32 * 64 * 128 * 4 + 8 * 32 * 64 * 2 * 4
    n = fd.workspace_bytes("fd_decode_attn", B=1, Hq=1, Hkv=1, L=1, d=64, chunk=16)
    assert n == 512
    # 12 units of 64 positions: the call's split halves to 32 (a multiple of
    # the page), 5 chunks per sequence
    n = fd.workspace_bytes("fd_decode_attn_paged", B=2, Hq=8, Hkv=2, d=128, page=16,
                           max_pages=10, max_seq_len=160, chunk=64)
    assert n == 2 * 8 * 5 * 128 * 4 + 768      # 640 B of (m, l) rounded up to 768
    # pages of 64: the split stays at the chunk
    n = fd.workspace_bytes("fd_decode_attn_paged", B=2, Hq=8, Hkv=2, d=128, page=64,
                           max_pages=10, max_seq_len=160, chunk=64)
    assert n == 2 * 8 * 3 * 128 * 4 + 512      # 384 B of (m, l) rounded up to 512


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), _abi.FD_ERR_UNSUPPORTED),
    (dict(Hq=9), _abi.FD_ERR_ARG),             # not a multiple of Hkv
    (dict(Hq=32, Hkv=2, dt=_abi.FD_F32), _abi.FD_ERR_UNSUPPORTED),   # group of 16 in fp32
    (dict(Hq=7, Hkv=1, dt=_abi.FD_F32), _abi.FD_ERR_UNSUPPORTED),    # group of 7 in fp32
    (dict(Hq=66, Hkv=2), _abi.FD_ERR_UNSUPPORTED),                   # group of 33
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


@pytest.mark.parametrize("Hq,Hkv", [(28, 4), (48, 8), (32, 2), (32, 1), (3, 1), (12, 2)])
def test_any_group_up_to_32_on_bf16(Hq, Hkv):
    """Group sizes outside {1, 2, 4, 8} (7, 6, 16, 32, 3, 6) take the
    matrix-core kernel on bf16 inputs: the dense entry points accept them
    with the usual workspace; the paged, fixed-maximum and FFD entry points
    do not."""
    n = fd.workspace_bytes("fd_decode_attn", B=2, Hq=Hq, Hkv=Hkv, L=1000, d=128, chunk=64)
    assert n == 2 * Hq * 16 * 128 * 4 + -(-2 * Hq * 16 * 2 * 4 // 256) * 256
    assert fd.workspace_bytes("fd_decode_attn_multi", B=2, M=1, Hq=Hq, Hkv=Hkv, L=1000, d=128,
                              chunk=64) == n
    for entry, kw in [("fd_decode_attn_unified_max", dict(L=1000, chunk=64)),
                      ("fd_ffd_sparse_decode", dict(L=1000, chunk=64)),
                      ("fd_decode_attn_paged", dict(page=16, max_pages=64, max_seq_len=1000,
                                                    chunk=64))]:
        with pytest.raises(fd.FdError) as e:
            fd.workspace_bytes(entry, B=2, Hq=Hq, Hkv=Hkv, d=128, **kw)
        assert e.value.code == _abi.FD_ERR_UNSUPPORTED, entry


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


def test_ffd_pack_rejects_misaligned_zs():
    """The packer stores each (zero, step) pair as one 32-bit word, so zs must
    be 4-byte aligned, as fd_ffd_sparse_decode also requires.  The pointers
    are never dereferenced: validation fails first."""
    lib = fd.lib()
    p = C.c_void_p(256)
    assert lib.fd_ffd_pack(p, p, C.c_void_p(258), p, p, 1, 1, 16, 128, 0, 16,
                           None) == _abi.FD_ERR_ARG
    assert b"zs" in lib.fd_last_error()
    for args in [(p, p, C.c_void_p(258), p, p, p, p, p, 1, 8, 2, 64, 128, 0.1, 5.0, 4, 64, 32,
                  None, None, p, C.byref(C.c_size_t(1 << 30)), None)]:
        assert lib.fd_ffd_sparse_decode(*args) == _abi.FD_ERR_ARG


def test_multi_paged_validation_and_workspace():
    base = dict(B=3, M=4, Hq=8, Hkv=2, d=128, page=16, max_pages=8, max_seq_len=100, chunk=32)

    def a256(x):
        return -(-x // 256) * 256

    def slots(S, R=16, d=128):   # worker slots: S*R*d and S*R*2 floats, S*4 int32, one word
        return a256(S * R * d * 4) + a256(S * R * 2 * 4) + a256(S * 16) + 256
    # partials of B*M*Hq rows over ceil(100 / 32) = 4 chunks, then B*Hkv*4 = 24
    # worker slots of R = G*M = 16 rows
    assert fd.workspace_bytes("fd_decode_attn_multi_paged", **base) == \
        3 * 4 * 8 * 4 * 128 * 4 + 3 * 4 * 8 * 4 * 2 * 4 + slots(24)
    assert fd.workspace_bytes("fd_decode_attn_multi_paged", **dict(base, max_seq_len=0)) == \
        256 + slots(1)
    # 17-32 rows (the wave-pair kernel): slots of R = 32 rows
    assert fd.workspace_bytes("fd_decode_attn_multi_paged", **dict(base, M=8)) == \
        3 * 8 * 8 * 4 * 128 * 4 + 3 * 8 * 8 * 4 * 2 * 4 + slots(24, R=32)
    # the slots stop at 2,048 workers
    big = dict(base, B=64, Hkv=8, Hq=128, M=1, max_pages=8192, max_seq_len=131072, chunk=1024)
    nc = 128
    assert fd.workspace_bytes("fd_decode_attn_multi_paged", **big) == \
        a256(64 * 128 * nc * 128 * 4) + a256(64 * 128 * nc * 8) + slots(2048)
    for bad, code in [(dict(page=8, max_pages=16), _abi.FD_ERR_UNSUPPORTED),  # matrix path: pages >= 16
                      (dict(page=12), _abi.FD_ERR_ARG),
                      (dict(page=32, chunk=48), _abi.FD_ERR_ARG),       # not a multiple of the page
                      (dict(page=16, chunk=16 * 512, max_pages=600), _abi.FD_ERR_UNSUPPORTED),
                      (dict(max_seq_len=129), _abi.FD_ERR_ARG),         # beyond max_pages * page
                      (dict(M=9), _abi.FD_ERR_UNSUPPORTED),             # G*M = 36 rows
                      (dict(dt=_abi.FD_F32), _abi.FD_ERR_UNSUPPORTED),
                      (dict(M=0), _abi.FD_ERR_ARG)]:
        kw = dict(base); kw.update(bad)
        with pytest.raises(fd.FdError) as e:
            fd.workspace_bytes("fd_decode_attn_multi_paged", **kw)
        assert e.value.code == code, bad
    # one token of a vector-kernel group: the paged single-query path (pages of 8, fp32)
    assert fd.workspace_bytes("fd_decode_attn_multi_paged",
                              **dict(base, M=1, page=8, max_pages=16, dt=_abi.FD_F32)) > 0


def test_short_calls_take_shorter_splits():
    """fd_decode_attn halves the split of a call with fewer (sequence,
    kv-head, chunk) units than the 1,024 SIMDs, down to 32 positions, and
    sizes its workspace for that; fd_decode_attn_partials keeps one partial
    per chunk."""
    def size(B, Hq, n, d):
        return B * Hq * n * d * 4 + -(-(B * Hq * n * 8) // 256) * 256
    # 512 units -> splits of 256: 128 per sequence and kv-head
    assert fd.workspace_bytes("fd_decode_attn", B=1, Hq=32, Hkv=8, L=32768, d=128,
                              chunk=512) == size(1, 32, 128, 128)
    # the fp32 MHA workload: 32 units -> splits of 32 positions, 1,024 units
    assert fd.workspace_bytes("fd_decode_attn", dt=_abi.FD_F32, B=1, Hq=8, Hkv=8, L=4096, d=64,
                              chunk=1024) == size(1, 8, 128, 64)
    # enough units already: the caller's chunk
    assert fd.workspace_bytes("fd_decode_attn", B=2, Hq=32, Hkv=8, L=32768, d=128,
                              chunk=512) == size(2, 32, 64, 128)
    # a chunk that is not a multiple of 32 stays
    assert fd.workspace_bytes("fd_decode_attn", B=1, Hq=8, Hkv=8, L=4096, d=64,
                              chunk=48) == size(1, 8, 86, 64)
