"""MI355X-native single-query decode attention (split-KV Flash-Decoding).

Thin Python binding over the C ABI of ``include/fd.h``.  The functions here
only marshal arguments (shapes, dtypes, device pointers, the current HIP
stream); every step of the computation runs in the HIP kernels of
``libfd_amd.so``.  PyTorch supplies device memory and streams.

Entry points (names follow the C ABI):
  decode_attn            dense contiguous cache
  decode_attn_noalloc    the same without a workspace (library-owned buffer)
  decode_attn_partials, merge_partials   its two stages
  decode_attn_paged      paged cache with a block table
  decode_attn_unified_max  fixed maximum with exact fallback
  decode_attn_multi      several new query tokens per sequence (causal)
  kv_append, kv_append_paged   the step's new K/V rows into the cache
  ffd_pack               2-bit + 8-bit residual key format
  ffd_sparse_decode      FFD: 2-bit scan, pseudo-max, top-delta, refine
"""
from __future__ import annotations

import ctypes as C
import math

import torch

from . import _abi
from ._abi import FD_BF16, FD_F32, FdError  # noqa: F401

__all__ = ["decode_attn", "decode_attn_noalloc", "decode_attn_partials", "merge_partials", "partial_views",
           "decode_attn_paged", "decode_attn_unified_max", "decode_attn_multi", "kv_append",
           "kv_append_paged",
           "ffd_pack", "ffd_sparse_decode",
           "workspace_bytes", "FdError", "lib"]


def lib():
    return _abi.load()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FD_BF16
    if t.dtype == torch.float32:
        return FD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(dev) -> C.c_void_p:
    return C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, shape=None, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(fn, args, ws, dev):
    """Two-phase workspace: size query (ws = NULL), then allocate if needed."""
    need = C.c_size_t(0)
    _abi.check(fn(*args(None, C.byref(need))))
    if ws is None or ws.numel() < need.value:
        ws = torch.empty(max(need.value, 256), dtype=torch.uint8, device=dev)
    size = C.c_size_t(ws.numel())
    return ws, size


def _outs(B, Hq, d, dev, out, lse, want_lse):
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    _need(out, "out", (B, Hq, d), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, Hq), torch.float32, dev)
    return out, lse


def decode_attn(q, k, v, chunk=512, scale=None, out=None, lse=None, want_lse=True,
                workspace=None):
    """Dense decode attention: q [B,Hq,d], k/v [B,Hkv,L,d] (bf16 or fp32).
    Returns (out fp32 [B,Hq,d], lse fp32 [B,Hq] or None)."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, L, d,
                scale, int(chunk), ws, wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn, args, workspace, dev)
    _abi.check(L_.fd_decode_attn(*args(_ptr(workspace), C.byref(size))))
    return out, lse


def decode_attn_noalloc(q, k, v, chunk=512, scale=None, out=None, lse=None, want_lse=True):
    """decode_attn without a workspace: the chunk partials go to the library's
    own per-device buffer (FD_NOALLOC_BYTES); nothing is allocated when out
    (and lse, if wanted) are given.  Calls that overlap on one device race."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    _abi.check(lib().fd_decode_attn_noalloc(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                            _ptr(lse), B, Hq, Hkv, L, d, scale, int(chunk),
                                            _stream(dev)))
    return out, lse


def decode_attn_partials(q, k, v, chunk=512, scale=None, workspace=None):
    """First stage of decode_attn: chunk partials into ``workspace`` (uint8
    tensor, allocated if None or too small).  Returns (workspace, n_chunks)."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, L, d, scale, int(chunk), ws,
                wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn_partials, args, workspace, dev)
    _abi.check(L_.fd_decode_attn_partials(*args(_ptr(workspace), C.byref(size))))
    return workspace, (L + int(chunk) - 1) // int(chunk)


def partial_views(workspace, B, Hq, n_chunks, d):
    """(O [B,Hq,nc,d], ML [B,Hq,nc,2]) fp32 views of a partials workspace."""
    n_o = B * Hq * n_chunks * d
    off = ((n_o * 4 + 255) // 256) * 256
    o = workspace[:n_o * 4].view(torch.float32).view(B, Hq, n_chunks, d)
    ml = workspace[off:off + B * Hq * n_chunks * 8].view(torch.float32).view(B, Hq, n_chunks, 2)
    return o, ml


def merge_partials(o_part, ml_part, out=None, lse=None, want_lse=True):
    """Exact merge of chunk partials O [B,Hq,nc,d], ML [B,Hq,nc,2] (fp32)."""
    B, Hq, nc, d = o_part.shape
    dev = o_part.device
    _need(o_part, "o_part", dtype=torch.float32)
    _need(ml_part, "ml_part", (B, Hq, nc, 2), torch.float32, dev)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    _abi.check(lib().fd_merge_partials(_ptr(o_part), _ptr(ml_part), _ptr(out), _ptr(lse), B,
                                       Hq, nc, d, _stream(dev)))
    return out, lse


def decode_attn_paged(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, chunk=512,
                      scale=None, out=None, lse=None, want_lse=True, workspace=None):
    """Paged decode attention: pools [P,Hkv,page,d], block_table int32
    [B,max_pages], seq_lens int32 [B] (device), max_seq_len a host bound."""
    B, Hq, d = q.shape
    P, Hkv, page = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k_pool, "k_pool", (P, Hkv, page, d), q.dtype, dev)
    _need(v_pool, "v_pool", (P, Hkv, page, d), q.dtype, dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(seq_lens, "seq_lens", (B,), torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv, d, page,
                block_table.shape[1], P, int(max_seq_len), scale, int(chunk), ws, wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn_paged, args, workspace, dev)
    _abi.check(L_.fd_decode_attn_paged(*args(_ptr(workspace), C.byref(size))))
    return out, lse


def decode_attn_unified_max(q, k, v, phi, chunk=512, margin_hi=10.0, margin_lo=40.0,
                            scale=None, out=None, lse=None, want_lse=True, flags=None,
                            want_flags=True, workspace=None):
    """Fixed-maximum decode attention with exact fallback.
    Returns (out, lse, chunk_flags uint8 [B,Hq,n_chunks] or None)."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nc = (L + int(chunk) - 1) // int(chunk)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    if flags is None and want_flags:
        flags = torch.empty((B, Hq, nc), dtype=torch.uint8, device=dev)
    if flags is not None:
        _need(flags, "flags", (B, Hq, nc), torch.uint8, dev)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, L, d,
                scale, int(chunk), float(phi), float(margin_hi), float(margin_lo),
                _ptr(flags), ws, wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn_unified_max, args, workspace, dev)
    _abi.check(L_.fd_decode_attn_unified_max(*args(_ptr(workspace), C.byref(size))))
    return out, lse, flags


def decode_attn_multi(q, k, v, chunk=512, scale=None, out=None, lse=None, want_lse=True,
                      workspace=None):
    """Multi-row decode: q [B,M,Hq,d] (M new tokens whose K/V sit at positions
    L-M..L-1 of k/v [B,Hkv,L,d]); token r sees positions 0..L-M+r.
    Returns (out fp32 [B,M,Hq,d], lse fp32 [B,M,Hq] or None)."""
    B, M, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k, "k", (B, Hkv, L, d), q.dtype, dev)
    _need(v, "v", (B, Hkv, L, d), q.dtype, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, M, Hq, d), dtype=torch.float32, device=dev)
    _need(out, "out", (B, M, Hq, d), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, M, Hq), torch.float32, dev)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, M, Hq, Hkv, L, d,
                scale, int(chunk), ws, wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn_multi, args, workspace, dev)
    _abi.check(L_.fd_decode_attn_multi(*args(_ptr(workspace), C.byref(size))))
    return out, lse


def decode_attn_multi_paged(q, k_pool, v_pool, block_table, seq_lens, max_seq_len, chunk=512,
                            scale=None, out=None, lse=None, want_lse=True, workspace=None):
    """Multi-row decode over a paged cache: q [B,M,Hq,d], pools [P,Hkv,page,d],
    block_table int32 [B,max_pages], seq_lens int32 [B] (device; sequence b's M
    new tokens sit at seq_lens[b]-M..seq_lens[b]-1), max_seq_len a host bound.
    Returns (out fp32 [B,M,Hq,d], lse fp32 [B,M,Hq] or None)."""
    B, M, Hq, d = q.shape
    P, Hkv, page = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    dev = q.device
    _need(q, "q", device=dev)
    _need(k_pool, "k_pool", (P, Hkv, page, d), q.dtype, dev)
    _need(v_pool, "v_pool", (P, Hkv, page, d), q.dtype, dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(seq_lens, "seq_lens", (B,), torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, M, Hq, d), dtype=torch.float32, device=dev)
    _need(out, "out", (B, M, Hq, d), torch.float32, dev)
    if lse is None and want_lse:
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", (B, M, Hq), torch.float32, dev)
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_dt(q), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                _ptr(seq_lens), _ptr(out), _ptr(lse), B, M, Hq, Hkv, d, page,
                block_table.shape[1], P, int(max_seq_len), scale, int(chunk), ws, wsb, st)
    workspace, size = _workspace(L_.fd_decode_attn_multi_paged, args, workspace, dev)
    _abi.check(L_.fd_decode_attn_multi_paged(*args(_ptr(workspace), C.byref(size))))
    return out, lse


def kv_append(k_new, v_new, k_cache, v_cache, t):
    """Write k_new/v_new [B,Hkv,M,d] into rows t..t+M-1 of the contiguous
    caches [B,Hkv,L_cap,d] (same dtype)."""
    B, Hkv, M, d = k_new.shape
    L_cap = k_cache.shape[2]
    dev = k_new.device
    _need(k_new, "k_new", device=dev)
    _need(v_new, "v_new", (B, Hkv, M, d), k_new.dtype, dev)
    _need(k_cache, "k_cache", (B, Hkv, L_cap, d), k_new.dtype, dev)
    _need(v_cache, "v_cache", (B, Hkv, L_cap, d), k_new.dtype, dev)
    _abi.check(lib().fd_kv_append(_dt(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                  _ptr(v_cache), B, Hkv, M, L_cap, d, int(t), _stream(dev)))


def kv_append_paged(k_new, v_new, k_pool, v_pool, block_table, pos):
    """Write k_new/v_new [B,Hkv,M,d] at positions pos[b]..pos[b]+M-1 (pos int32
    [B], device) of the paged pools [P,Hkv,page,d] through block_table int32
    [B,max_pages]; positions without a valid page are skipped."""
    B, Hkv, M, d = k_new.shape
    P, page = k_pool.shape[0], k_pool.shape[2]
    dev = k_new.device
    _need(k_new, "k_new", device=dev)
    _need(v_new, "v_new", (B, Hkv, M, d), k_new.dtype, dev)
    _need(k_pool, "k_pool", (P, Hkv, page, d), k_new.dtype, dev)
    _need(v_pool, "v_pool", (P, Hkv, page, d), k_new.dtype, dev)
    _need(block_table, "block_table", dtype=torch.int32, device=dev)
    _need(pos, "pos", (B,), torch.int32, dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages]")
    _abi.check(lib().fd_kv_append_paged(_dt(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                        _ptr(v_pool), _ptr(block_table), _ptr(pos), B, Hkv, M,
                                        d, page, block_table.shape[1], P, _stream(dev)))


def ffd_pack(k, t_begin=0, t_end=None, out=None):
    """Quantise bf16 keys k [B,Hkv,L,d] into the FFD format.  Returns dict
    codes (int32 view of uint32 words), zs (fp16 bits as int16), res (int8),
    rs (fp16 bits as int16); with ``out`` given, fills positions
    [t_begin, t_end) of those arrays in place."""
    B, Hkv, L, d = k.shape
    dev = k.device
    _need(k, "k", dtype=torch.bfloat16)
    t_end = L if t_end is None else int(t_end)
    if out is None:
        out = dict(codes=torch.zeros((B, Hkv, L, d // 16), dtype=torch.int32, device=dev),
                   zs=torch.zeros((B, Hkv, L, d // 32, 2), dtype=torch.int16, device=dev),
                   res=torch.zeros((B, Hkv, L, d), dtype=torch.int8, device=dev),
                   rs=torch.zeros((B, Hkv, L, d // 32), dtype=torch.int16, device=dev))
    _need(out["codes"], "codes", (B, Hkv, L, d // 16), torch.int32, dev)
    _need(out["zs"], "zs", (B, Hkv, L, d // 32, 2), torch.int16, dev)
    _need(out["res"], "res", (B, Hkv, L, d), torch.int8, dev)
    _need(out["rs"], "rs", (B, Hkv, L, d // 32), torch.int16, dev)
    _abi.check(lib().fd_ffd_pack(_ptr(k), _ptr(out["codes"]), _ptr(out["zs"]),
                                 _ptr(out["res"]), _ptr(out["rs"]), B, Hkv, L, d,
                                 int(t_begin), t_end, _stream(dev)))
    return out


def ffd_sparse_decode(q, packed, v, delta, n_sink=4, n_local=64, chunk=1024, scale=None,
                      out=None, lse=None, want_lse=True, want_mask=False,
                      want_pseudo_max=False, workspace=None):
    """FFD sparse decode.  q bf16 [B,Hq,d]; packed = dict from ffd_pack (or
    the same arrays built elsewhere); v bf16 [B,Hkv,L,d].
    Returns (out, lse, cand_mask int32 [B,Hq,ceil(L/32)] or None,
    pseudo_max fp32 [B,Hq] or None)."""
    B, Hq, d = q.shape
    Hkv, L = v.shape[1], v.shape[2]
    dev = q.device
    _need(q, "q", dtype=torch.bfloat16, device=dev)
    _need(v, "v", (B, Hkv, L, d), torch.bfloat16, dev)
    _need(packed["codes"], "codes", (B, Hkv, L, d // 16), torch.int32, dev)
    _need(packed["zs"], "zs", (B, Hkv, L, d // 32, 2), torch.int16, dev)
    _need(packed["res"], "res", (B, Hkv, L, d), torch.int8, dev)
    _need(packed["rs"], "rs", (B, Hkv, L, d // 32), torch.int16, dev)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outs(B, Hq, d, dev, out, lse, want_lse)
    mask = torch.empty((B, Hq, (L + 31) // 32), dtype=torch.int32, device=dev) \
        if want_mask else None
    pmax = torch.empty((B, Hq), dtype=torch.float32, device=dev) if want_pseudo_max else None
    L_ = lib()
    st = _stream(dev)

    def args(ws, wsb):
        return (_ptr(q), _ptr(packed["codes"]), _ptr(packed["zs"]), _ptr(packed["res"]),
                _ptr(packed["rs"]), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, L, d, scale,
                float(delta), int(n_sink), int(n_local), int(chunk), _ptr(mask), _ptr(pmax),
                ws, wsb, st)
    workspace, size = _workspace(L_.fd_ffd_sparse_decode, args, workspace, dev)
    _abi.check(L_.fd_ffd_sparse_decode(*args(_ptr(workspace), C.byref(size))))
    return out, lse, mask, pmax


def workspace_bytes(entry: str, **kw) -> int:
    """Workspace size an entry point needs (no GPU work): e.g.
    workspace_bytes('fd_decode_attn', B=8, Hq=32, Hkv=8, L=32768, d=128, chunk=512)."""
    L_ = lib()
    need = C.c_size_t(0)
    g = kw.get
    if entry == "fd_decode_attn":
        rc = L_.fd_decode_attn(g("dt", FD_BF16), None, None, None, None, None, g("B"),
                               g("Hq"), g("Hkv"), g("L"), g("d"), g("scale", 0.1),
                               g("chunk"), None, C.byref(need), None)
    elif entry == "fd_decode_attn_multi":
        rc = L_.fd_decode_attn_multi(g("dt", FD_BF16), None, None, None, None, None, g("B"),
                                     g("M"), g("Hq"), g("Hkv"), g("L"), g("d"), g("scale", 0.1),
                                     g("chunk"), None, C.byref(need), None)
    elif entry == "fd_decode_attn_multi_paged":
        rc = L_.fd_decode_attn_multi_paged(g("dt", FD_BF16), None, None, None, None, None,
                                           None, None, g("B"), g("M"), g("Hq"), g("Hkv"),
                                           g("d"), g("page", 16), g("max_pages"),
                                           g("num_pages", 1), g("max_seq_len"),
                                           g("scale", 0.1), g("chunk"), None, C.byref(need),
                                           None)
    elif entry == "fd_decode_attn_unified_max":
        rc = L_.fd_decode_attn_unified_max(g("dt", FD_BF16), None, None, None, None, None,
                                           g("B"), g("Hq"), g("Hkv"), g("L"), g("d"),
                                           g("scale", 0.1), g("chunk"), g("phi", 0.0),
                                           g("margin_hi", 10.0), g("margin_lo", 40.0), None,
                                           None, C.byref(need), None)
    elif entry == "fd_decode_attn_paged":
        rc = L_.fd_decode_attn_paged(g("dt", FD_BF16), None, None, None, None, None, None,
                                     None, g("B"), g("Hq"), g("Hkv"), g("d"), g("page", 16),
                                     g("max_pages"), g("num_pages", 1), g("max_seq_len"),
                                     g("scale", 0.1), g("chunk"), None, C.byref(need), None)
    elif entry == "fd_ffd_sparse_decode":
        rc = L_.fd_ffd_sparse_decode(None, None, None, None, None, None, None, None, g("B"),
                                     g("Hq"), g("Hkv"), g("L"), g("d"), g("scale", 0.1),
                                     g("delta", 5.0), g("n_sink", 4), g("n_local", 64),
                                     g("chunk"), None, None, None, C.byref(need), None)
    else:
        raise ValueError(entry)
    _abi.check(rc)
    return need.value
