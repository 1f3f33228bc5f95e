"""GPU parity of the dense split-KV path against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import flash_decoding as ofd
from tests.helpers import TOL, banner, f64, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(c, chunk=None, tol=None):
    chunk = c.chunk if chunk is None else chunk
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = ofd.dense_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    tol = TOL[c.q.dtype] if tol is None else tol
    eo, el = max_err(f64(out), ref), max_err(f64(lse), lref)
    assert eo <= tol and el <= tol, (eo, el)
    return out, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_shapes_groups_dtypes(dtype, d, G):
    banner(f"dense dtype={dtype} d={d} G={G}")
    c = W.dense_case(2, 8 if G < 8 else 16, (8 if G < 8 else 16) // G, 1000, d, dtype, 256,
                     seed=10 + G, device=DEV)
    _check(c)


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 255, 256, 257, 511, 512, 513, 4097])
def test_lengths_around_chunk_edges(L):
    banner(f"dense L={L}")
    _check(W.dense_case(2, 8, 2, L, 128, "bf16", 256, seed=L, device=DEV))


def test_config1_fp32_mha():
    banner("dense config1 fp32")
    _check(W.config_case(1, device=DEV))


@pytest.mark.parametrize("chunk", [16, 48, 128, 512, 4096])
def test_chunk_independence(chunk):
    banner(f"dense chunk={chunk}")
    c = W.dense_case(1, 8, 2, 3000, 128, "f32", 512, seed=5, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=chunk)
    ref, lref = fd.decode_attn(c.q, c.k, c.v, chunk=3008)   # one chunk
    assert max_err(f64(out), f64(ref)) < 1e-5 and max_err(f64(lse), f64(lref)) < 1e-5
    _check(c, chunk=chunk)


def test_single_key_is_value_bitwise():
    c = W.dense_case(2, 8, 8, 1, 64, "f32", 16, seed=3, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=16)
    torch.cuda.synchronize()
    assert torch.equal(out, c.v[:, :, 0].float())


def test_zero_query_is_mean():
    c = W.dense_case(1, 4, 4, 777, 128, "f32", 64, seed=4, device=DEV)
    q = torch.zeros_like(c.q)
    out, lse = fd.decode_attn(q, c.k, c.v, chunk=64)
    assert max_err(f64(out), f64(c.v).mean(2)) < 1e-5
    assert max_err(f64(lse), np.full((1, 4), math.log(777))) < 1e-5


def test_large_shift_no_overflow():
    # scores around +1000: the running maximum keeps exp finite
    c = W.dense_case(1, 4, 1, 2000, 64, "f32", 128, seed=6, device=DEV)
    qd = f64(c.q)[0, 0]
    w = 1000.0 * qd / (c.scale * (qd @ qd))
    k = c.k + torch.as_tensor(w, dtype=torch.float32, device=DEV)
    out, lse = fd.decode_attn(c.q[:, :1].contiguous(), k, c.v, chunk=128)
    ref, lref = ofd.dense_attention(f64(c.q)[:, :1], f64(k), f64(c.v), c.scale)
    assert np.all(np.isfinite(f64(out)))
    assert max_err(f64(out), ref) < 1e-4 and max_err(f64(lse), lref) < 1e-3


def test_deterministic_bitwise():
    c = W.dense_case(2, 32, 8, 5000, 128, "bf16", 512, seed=7, device=DEV)
    a, la = fd.decode_attn(c.q, c.k, c.v, chunk=512)
    b, lb = fd.decode_attn(c.q, c.k, c.v, chunk=512)
    assert torch.equal(a, b) and torch.equal(la, lb)


def _check_every_row(c, out, lse, tol=2e-3):
    """Every (sequence, head) of a large case against the oracle, one
    sequence at a time (bounded host memory)."""
    assert torch.isfinite(out).all()
    for b in range(c.q.shape[0]):
        ref, lref = ofd.dense_attention(f64(c.q[b:b + 1]), f64(c.k[b:b + 1]), f64(c.v[b:b + 1]),
                                        c.scale)
        eo, el = max_err(f64(out[b:b + 1]), ref), max_err(f64(lse[b:b + 1]), lref)
        assert eo <= tol and el <= tol, (b, eo, el)


def test_config2_full_size():
    """Headline workload (B 8, Hq 32, Hkv 8, d 128, L 32768, chunk 512):
    every one of the 256 (sequence, head) rows."""
    banner("dense config2 full size")
    c = W.config_case(2, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=c.chunk)
    torch.cuda.synchronize()
    _check_every_row(c, out, lse)


def test_dense_128k():
    """The long end of the 32K-128K range: B 2, L 131072, chunk 512 (256
    chunks per row: the merge with its columns over 8 wavefronts, four
    chunks' (m, l) per lane)."""
    banner("dense 128K")
    c = W.dense_case(2, 32, 8, 131072, 128, "bf16", 512, seed=1202, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=c.chunk)
    torch.cuda.synchronize()
    _check_every_row(c, out, lse)


def test_many_units_per_wave():
    """Chunks of 16 over L 65536: 131,072 units, 128 per wave, so every wave
    writes its held partials many times mid-run, and the merge walks 4,096
    chunks per row in tiles of 256."""
    banner("dense many units per wave")
    c = W.dense_case(4, 32, 8, 65536, 128, "bf16", 16, seed=1203, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=c.chunk)
    torch.cuda.synchronize()
    _check_every_row(c, out, lse)


def test_partials_then_merge_equals_full_call():
    """With at least 1,024 units the full call keeps the caller's chunk, so
    its two stages give it bit for bit."""
    c = W.dense_case(8, 32, 8, 4100, 128, "bf16", 256, seed=41, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=256)
    ws, nc = fd.decode_attn_partials(c.q, c.k, c.v, chunk=256)
    o_part, ml_part = fd.partial_views(ws, 8, 32, nc, 128)
    out2, lse2 = fd.merge_partials(o_part, ml_part)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_short_call_splits_match_the_chunked_stages(dt, d):
    """A call of few units (B 1, 8 kv-heads) takes shorter splits than its
    chunk; its result equals the chunk's partials merged, to fp32 rounding,
    and the oracle."""
    banner(f"dense short call {dt} d={d}")
    c = W.dense_case(1, 32 if d == 128 else 8, 8, 3000, d, dt, 512, seed=44, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=512)
    ws, nc = fd.decode_attn_partials(c.q, c.k, c.v, chunk=512)
    o_part, ml_part = fd.partial_views(ws, 1, c.q.shape[1], nc, d)
    out2, lse2 = fd.merge_partials(o_part, ml_part)
    torch.cuda.synchronize()
    assert max_err(f64(out), f64(out2)) <= 1e-6 and max_err(f64(lse), f64(lse2)) <= 1e-6
    _check(c, chunk=512)


def test_merge_independent_of_chunk_order():
    c = W.dense_case(1, 8, 2, 4000, 64, "f32", 128, seed=42, device=DEV)
    ws, nc = fd.decode_attn_partials(c.q, c.k, c.v, chunk=128)
    o_part, ml_part = fd.partial_views(ws, 1, 8, nc, 64)
    ref, lref = fd.merge_partials(o_part.clone(), ml_part.clone())
    perm = torch.randperm(nc, generator=torch.Generator().manual_seed(3)).to(DEV)
    out, lse = fd.merge_partials(o_part[:, :, perm].contiguous(), ml_part[:, :, perm].contiguous())
    assert max_err(f64(out), f64(ref)) < 1e-6 and max_err(f64(lse), f64(lref)) < 1e-6


def test_sequence_split_merged_from_two_halves():
    # Two devices' worth of a sequence-parallel split, on one GPU: partials of
    # each half of the cache, gathered along the chunk axis, one merge.
    c = W.dense_case(2, 32, 8, 4096, 128, "bf16", 512, seed=43, device=DEV)
    parts = []
    for lo, hi in ((0, 2048), (2048, 4096)):
        k = c.k[:, :, lo:hi].contiguous()
        v = c.v[:, :, lo:hi].contiguous()
        ws, nc = fd.decode_attn_partials(c.q, k, v, chunk=512)
        parts.append([t.clone() for t in fd.partial_views(ws, 2, 32, nc, 128)])
    o = torch.cat([p[0] for p in parts], dim=2).contiguous()
    ml = torch.cat([p[1] for p in parts], dim=2).contiguous()
    out, lse = fd.merge_partials(o, ml)
    ref, lref = ofd.dense_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3


@pytest.mark.parametrize("d", [64, 128])
def test_merge_of_many_chunks(d):
    """Rows of 257 chunks take the workgroup merge and cross its 256-chunk
    weight tile."""
    banner(f"dense many chunks d={d}")
    c = W.dense_case(2, 8, 2, 16 * 256 + 5, d, "bf16", 16, seed=41 + d, device=DEV)
    _check(c)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nc", [1, 2, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257])
def test_merge_tier_edges(d, nc):
    """Each side of every merge tier: rows of up to 256 chunks on single
    wavefronts, the columns split over more of them as rows grow (d 128: 1
    up to 32 chunks, 2 up to 64, 4 up to 128, 8 up to 256; d 64: 1 up to 64,
    2 up to 128, 4 up to 256), longer rows on 4-wave workgroups; the last
    chunk is ragged."""
    banner(f"dense merge tiers d={d} nc={nc}")
    c = W.dense_case(2, 8, 2, 16 * (nc - 1) + 7, d, "bf16", 16, seed=300 + nc + d, device=DEV)
    _check(c)


def test_dense_one_million_positions():
    """One sequence of 2^20 + 77 positions (512 MiB of K/V): 2,049 chunks of
    512 with a ragged last one, so the merge walks 9 tiles of 256 chunks, the
    last holding a single chunk.  Every head checked."""
    banner("dense 1M")
    L = (1 << 20) + 77
    c = W.dense_case(1, 8, 1, L, 128, "bf16", 512, seed=1204, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=c.chunk)
    torch.cuda.synchronize()
    _check_every_row(c, out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_group_of_eight_long_calls(dtype, d):
    """G = 8 on a call of 1,024 (sequence, kv-head, chunk) units: bf16 runs on
    the matrix-core kernel, fp32 on the vector kernel; every row against the
    oracle, and the partials entry point merged gives the same rows."""
    banner(f"dense G=8 long call {dtype} d={d}")
    c = W.dense_case(8, 64, 8, 8192 - 5, d, dtype, 512, seed=1300 + d, device=DEV)
    out, _ = _check(c)
    ws, nc = fd.decode_attn_partials(c.q, c.k, c.v, chunk=512)
    o_part, ml_part = fd.partial_views(ws, 8, 64, nc, d)
    out2, lse2 = fd.merge_partials(o_part, ml_part)
    torch.cuda.synchronize()
    ref, lref = ofd.dense_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    assert max_err(f64(out2), ref) <= TOL[c.q.dtype]
    assert max_err(f64(lse2), lref) <= TOL[c.q.dtype]
