"""fd_decode_attn_noalloc (library-owned partials buffer, no workspace, no
allocation) against fd_decode_attn, which runs the same kernels on a caller
workspace: bitwise equal, and within the parity bar of the fp64 oracle, on
calls in a row, each with a smaller input than the one before."""
import ctypes as C

import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from long_context_decode_fd_amd import _abi
from oracle import flash_decoding as ofd
from tests.helpers import TOL, banner, f64, max_err

DEV = "cuda:0"


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    cases = [
        # largest first: eight heads per kv-head on 1,024 units, which runs on
        # the matrix-core kernel (B 8, Hq 64, Hkv 8, d 128, L 8187)
        (8, 64, 8, 8187, 128, "bf16", 512, 73),
        # B 4, Hq 32, Hkv 8, d 128, L 20000 (40 chunks of 512, ragged)
        (4, 32, 8, 20000, 128, "bf16", 512, 71),
        # then smaller, another dtype and head size: what the first call left
        # in the buffer must not leak into this one
        (2, 8, 2, 3000, 64, "f32", 256, 72),
    ]
    for B, Hq, Hkv, L, d, dt, chunk, seed in cases:
        banner(f"noalloc B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} {dt} chunk={chunk}")
        c = W.dense_case(B, Hq, Hkv, L, d, dt, chunk, seed=seed, device=DEV)
        out_w, lse_w = fd.decode_attn(c.q, c.k, c.v, chunk=chunk)
        out_n = torch.full_like(out_w, float("nan"))
        lse_n = torch.full_like(lse_w, float("nan"))
        fd.decode_attn_noalloc(c.q, c.k, c.v, chunk=chunk, out=out_n, lse=lse_n)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: the same bits
        assert torch.equal(out_n, out_w) and torch.equal(lse_n, lse_w)
        ref, lref = ofd.dense_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
        tol = TOL[c.q.dtype]
        assert max_err(f64(out_n), ref) <= tol and max_err(f64(lse_n), lref) <= tol


def test_noalloc_rejects_partials_beyond_its_buffer_without_a_gpu():
    """Sizes are checked before anything touches a device: 8 x 32 heads x 512
    chunks of 16 x (128 + 2) floats = 68 MB of partials exceed the 32 MiB
    buffer (FD_ERR_WORKSPACE); NULL pointers are FD_ERR_ARG.  The pointers
    below are never dereferenced."""
    lib = fd.lib()
    p = C.c_void_p(256)
    rc = lib.fd_decode_attn_noalloc(1, p, p, p, p, None, 8, 32, 8, 8192, 128, 0.088, 16, None)
    assert rc == _abi.FD_ERR_WORKSPACE
    assert b"exceed" in lib.fd_last_error()
    # the largest headline-shaped call that fits: 8 x 32 x 252 chunks of 130 floats
    assert 8 * 32 * 252 * 130 * 4 <= _abi.FD_NOALLOC_BYTES < 8 * 32 * 253 * 130 * 4
    rc = lib.fd_decode_attn_noalloc(1, None, p, p, p, None, 8, 32, 8, 32768, 128, 0.088, 512,
                                    None)
    assert rc == _abi.FD_ERR_ARG
