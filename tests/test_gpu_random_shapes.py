"""Seeded random shapes through every attention entry point against the fp64
oracle.  Each case draws batch, kv-heads, group size, head dim, dtype,
length, chunk (and page, margins, anchors, delta where they apply), so that
combinations the hand-picked cases miss still meet the parity bar."""
import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import ffd as offd
from oracle import flash_decoding as ofd
from oracle import multi_row as omr
from oracle import paged as opg
from tests.helpers import TOL, banner, f64, max_err, packed_to_device
from tests.test_gpu_ffd import _check_all
from tests.test_gpu_paged_unified import _unified_check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N = 10


def _heads(rs):
    d = int(rs.choice([64, 128]))
    G = int(rs.choice([1, 2, 4, 8]))
    Hkv = int(rs.integers(1, 4))
    B = int(rs.integers(1, 5))
    return B, G * Hkv, Hkv, G, d


@pytest.mark.parametrize("i", range(N))
def test_dense_random(i):
    rs = np.random.default_rng(5000 + i)
    B, Hq, Hkv, G, d = _heads(rs)
    L = int(rs.integers(1, 3001))
    chunk = 16 * int(rs.integers(1, 65))
    dtype = str(rs.choice(["bf16", "f32"]))
    banner(f"random dense B={B} Hq={Hq} Hkv={Hkv} d={d} L={L} chunk={chunk} {dtype}")
    c = W.dense_case(B, Hq, Hkv, L, d, dtype, chunk, seed=5000 + i, device=DEV)
    out, lse = fd.decode_attn(c.q, c.k, c.v, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = ofd.dense_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    tol = TOL[c.q.dtype]
    assert max_err(f64(out), ref) <= tol and max_err(f64(lse), lref) <= tol


@pytest.mark.parametrize("i", range(N))
def test_paged_random(i):
    rs = np.random.default_rng(6000 + i)
    B, Hq, Hkv, G, d = _heads(rs)
    page = int(rs.choice([8, 16, 32, 64]))
    unit = max(page, 16)
    chunk = unit * int(rs.integers(1, max(2, 1024 // unit) + 1))
    lens = rs.integers(0, 2001, size=B)
    lens[rs.random(B) < 0.2] = 0
    dtype = torch.float32 if rs.random() < 0.3 else torch.bfloat16
    banner(f"random paged B={B} Hq={Hq} Hkv={Hkv} d={d} page={page} chunk={chunk} "
           f"lens={lens.tolist()} {dtype}")
    c = W.paged_case(B, Hq, Hkv, d, 0, 2000, page=page, chunk=chunk, seed=6000 + i,
                     device=DEV, lens=lens)
    if dtype == torch.float32:
        c.q, c.k_pool, c.v_pool = c.q.float(), c.k_pool.float(), c.v_pool.float()
    out, lse = fd.decode_attn_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                    int(max(lens.max(), 1)), chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = opg.paged_attention(f64(c.q), f64(c.k_pool), f64(c.v_pool),
                                    c.block_table.cpu().numpy(), c.seq_lens.cpu().numpy(),
                                    page, c.scale)
    assert max_err(f64(out), ref) <= TOL[dtype] and max_err(f64(lse), lref) <= TOL[dtype]


@pytest.mark.parametrize("i", range(N))
def test_unified_random(i):
    rs = np.random.default_rng(7000 + i)
    B, Hq, Hkv, G, d = _heads(rs)
    L = int(rs.integers(1, 3001))
    chunk = 16 * int(rs.integers(1, 65))
    dtype = str(rs.choice(["bf16", "f32"]))
    phi = float(rs.uniform(-4.0, 8.0))
    hi, lo = float(rs.uniform(0.5, 12.0)), float(rs.uniform(0.5, 40.0))
    banner(f"random unified B={B} Hq={Hq} Hkv={Hkv} d={d} L={L} chunk={chunk} {dtype} "
           f"phi={phi:.3f} +{hi:.2f}/-{lo:.2f}")
    c = W.dense_case(B, Hq, Hkv, L, d, dtype, chunk, seed=7000 + i, device=DEV)
    _unified_check(c, phi, hi, lo)


@pytest.mark.parametrize("i", range(N))
def test_multi_random(i):
    rs = np.random.default_rng(8000 + i)
    B, Hq, Hkv, G, d = _heads(rs)
    M = int(rs.integers(1, 32 // G + 1))
    L = int(rs.integers(M, 2501))
    chunk = 16 * int(rs.integers(1, 65))
    banner(f"random multi B={B} M={M} Hq={Hq} Hkv={Hkv} d={d} L={L} chunk={chunk}")
    c = W.multi_case(B, M, Hq, Hkv, L, d, chunk, seed=8000 + i, device=DEV)
    out, lse = fd.decode_attn_multi(c.q, c.k, c.v, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = omr.multi_row_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    tol = TOL[torch.bfloat16]
    assert max_err(f64(out), ref) <= tol and max_err(f64(lse), lref) <= tol


@pytest.mark.parametrize("i", range(N))
def test_any_group_random(i):
    """Group sizes drawn from 1-32 (most outside {1, 2, 4, 8}) with as many
    tokens as fit 32 query rows, through the multi-row entry point and, for
    one token, the single-query one."""
    rs = np.random.default_rng(8500 + i)
    G = int(rs.integers(1, 33))
    M = int(rs.integers(1, 32 // G + 1))
    Hkv, B = int(rs.integers(1, 4)), int(rs.integers(1, 5))
    d = int(rs.choice([64, 128]))
    L = int(rs.integers(M, 2501))
    chunk = 16 * int(rs.integers(1, 65))
    banner(f"random any-group B={B} M={M} G={G} Hkv={Hkv} d={d} L={L} chunk={chunk}")
    c = W.multi_case(B, M, G * Hkv, Hkv, L, d, chunk, seed=8500 + i, device=DEV)
    out, lse = fd.decode_attn_multi(c.q, c.k, c.v, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = omr.multi_row_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    tol = TOL[torch.bfloat16]
    assert max_err(f64(out), ref) <= tol and max_err(f64(lse), lref) <= tol
    if M == 1:
        o1, l1 = fd.decode_attn(c.q[:, 0].contiguous(), c.k, c.v, chunk=chunk)
        torch.cuda.synchronize()
        assert max_err(f64(o1), ref[:, 0]) <= tol and max_err(f64(l1), lref[:, 0]) <= tol


@pytest.mark.parametrize("i", range(N))
def test_multi_paged_random(i):
    """Several tokens (or a group outside {1, 2, 4, 8}) over a paged cache:
    group 1-32, tokens as fit 32 query rows, pages 16-128, chunks of 1-8
    pages, ragged lengths with empty and shorter-than-M sequences."""
    rs = np.random.default_rng(8700 + i)
    G = int(rs.integers(1, 33))
    M = int(rs.integers(1, 32 // G + 1))
    Hkv, B = int(rs.integers(1, 4)), int(rs.integers(1, 6))
    d = int(rs.choice([64, 128]))
    page = int(rs.choice([16, 32, 64, 128]))
    chunk = page * int(rs.integers(1, 9))
    lens = rs.integers(0, 2001, size=B)
    lens[rs.random(B) < 0.2] = 0
    lens[rs.random(B) < 0.2] = int(rs.integers(0, M + 1))
    banner(f"random multi paged B={B} M={M} G={G} Hkv={Hkv} d={d} page={page} chunk={chunk} "
           f"lens={lens.tolist()}")
    c = W.paged_case(B, G * Hkv, Hkv, d, 0, 2000, page=page, chunk=chunk, seed=8700 + i,
                     device=DEV, lens=lens, M=M)
    mx = int(lens.max())
    out, lse = fd.decode_attn_multi_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                          mx, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = opg.paged_multi_row_attention(
        f64(c.q), c.k_pool.float().cpu().numpy(), c.v_pool.float().cpu().numpy(),
        c.block_table.cpu().numpy(), lens, page, c.scale)
    tol = TOL[torch.bfloat16]
    assert max_err(f64(out), ref) <= tol and max_err(f64(lse), lref) <= tol


@pytest.mark.parametrize("i", range(N))
def test_ffd_random(i):
    rs = np.random.default_rng(9000 + i)
    B, Hq, Hkv, G, d = _heads(rs)
    L = int(rs.integers(1, 2501))
    cmax = 1024 if G == 8 else 2048
    chunk = 32 * int(rs.integers(1, cmax // 32 + 1))
    n_sink, n_local = int(rs.integers(0, 9)), int(rs.integers(0, 80))
    if n_sink + n_local == 0:
        n_local = 1
    delta = float(rs.choice([0.5, 3.0, 5.0, 7.0]))
    banner(f"random ffd B={B} Hq={Hq} Hkv={Hkv} d={d} L={L} chunk={chunk} "
           f"sinks={n_sink} local={n_local} delta={delta}")
    c = W.ffd_case(B, Hq, Hkv, L, d, n_sink=n_sink, n_local=n_local, chunk=chunk,
                   seed=9000 + i, device=DEV)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, packed_to_device(ph, DEV), c.v, delta,
                                                n_sink, n_local, chunk=chunk, want_mask=True,
                                                want_pseudo_max=True)
    torch.cuda.synchronize()
    _check_all(f64(c.q), ph, f64(c.v), G, c.scale, delta, n_sink, n_local, f64(out), f64(lse),
               cand.cpu().numpy().view(np.uint32), f64(pmax))
