"""GPU parity of multi-row decode (M new query tokens per sequence, causal
among them; matrix-core kernel) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import multi_row as omr
from tests.helpers import TOL, banner, f64, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOLB = TOL[torch.bfloat16]


def _check(c, chunk, rows=None):
    out, lse = fd.decode_attn_multi(c.q, c.k, c.v, chunk=chunk)
    torch.cuda.synchronize()
    ref, lref = omr.multi_row_attention(f64(c.q), f64(c.k), f64(c.v), c.scale, rows=rows)
    if rows is None:
        assert max_err(f64(out), ref) <= TOLB
        assert max_err(f64(lse), lref) <= TOLB
    else:
        for b, r, h in rows:
            assert max_err(f64(out[b, r, h]), ref[b, r, h]) <= TOLB, (b, r, h)
            assert abs(float(lse[b, r, h]) - lref[b, r, h]) <= TOLB, (b, r, h)
    assert torch.isfinite(out).all()
    return out, lse


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("G,M", [(4, 4), (4, 2), (4, 3), (8, 2), (2, 8), (1, 16), (1, 5),
                                 (8, 4), (4, 8), (2, 12), (1, 20), (8, 3)])
def test_multi_row_small(d, G, M):
    banner(f"multi d={d} G={G} M={M}")
    Hkv = 2
    # L spans several chunks and a ragged tail; batches of 64 positions too
    c = W.multi_case(2, M, G * Hkv, Hkv, 333, d, seed=100 + G * M + d, device=DEV)
    _check(c, chunk=128)


@pytest.mark.parametrize("L,M,chunk", [(4, 4, 16), (17, 4, 16), (64, 4, 64), (65, 4, 64),
                                       (1000, 3, 16)])
def test_multi_row_causal_edges(L, M, chunk):
    # L = M: the first token sees only position 0; chunks that lie wholly
    # beyond some tokens' last visible position
    c = W.multi_case(1, M, 8, 2, L, 128, seed=7 + L, device=DEV)
    _check(c, chunk=chunk)


def test_multi_row_one_token_is_single_query_decode():
    c = W.multi_case(2, 1, 8, 2, 500, 128, seed=3, device=DEV)
    out, lse = fd.decode_attn_multi(c.q, c.k, c.v, chunk=64)
    o2, l2 = fd.decode_attn(c.q[:, 0].contiguous(), c.k, c.v, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 0], o2) and torch.equal(lse[:, 0], l2)


def test_multi_row_peaked_scores():
    # sharp softmax (q x 6): p near 1 on few positions, the case where bf16
    # weights alone would miss 2e-3; the hi + lo split keeps it
    c = W.multi_case(2, 4, 8, 2, 2000, 128, seed=9, device=DEV, q_scale=6.0)
    _check(c, chunk=256)


def test_multi_row_chunk_independence():
    c = W.multi_case(1, 4, 8, 2, 3000, 128, seed=11, device=DEV)
    o1, l1 = fd.decode_attn_multi(c.q, c.k, c.v, chunk=64)
    o2, l2 = fd.decode_attn_multi(c.q, c.k, c.v, chunk=1024)
    torch.cuda.synchronize()
    assert max_err(f64(o1), f64(o2)) <= 1e-5 and max_err(f64(l1), f64(l2)) <= 1e-5


def test_multi_row_full_size():
    """Headline shape with four new tokens per sequence (G*M = 16 rows):
    every (sequence, token, head) row."""
    banner("multi full size B=8 L=32768 M=4")
    c = W.multi_case(8, 4, 32, 8, 32768, 128, seed=102, device=DEV)
    _check(c, chunk=512)


def test_multi_row_two_query_tiles_full_size():
    """Headline shape with eight new tokens per sequence (G*M = 32 rows: a
    pair of waves, one query tile each, sharing every K and V tile through
    LDS): every row.  64 chunks of 512 per row fold into splits of 4."""
    banner("multi full size B=8 L=32768 M=8")
    c = W.multi_case(8, 8, 32, 8, 32768, 128, seed=108, device=DEV)
    _check(c, chunk=512)


# The remaining large multi-row cases check a sample of rows: the oracle
# streams a row's whole fp64 K and V prefix for every row (64 MB per row at
# L 32768, 2 GB at 2^20), so every row would take minutes of host time; the
# two headline-shape tests above check every row.
def test_multi_row_small_chunks_folded_sampled():
    """Chunks of 32 at the headline shape: 1,024 chunks per row, folded into
    splits of 64 chunks (one split per wave slot)."""
    banner("multi full size B=8 L=32768 M=4 chunk=32")
    c = W.multi_case(8, 4, 32, 8, 32768, 128, seed=103, device=DEV)
    rows = [(0, 0, 0), (1, 3, 31), (4, 2, 9), (6, 1, 20), (7, 3, 2)]
    _check(c, chunk=32, rows=rows)


def test_multi_row_small_chunks_two_query_tiles_sampled():
    """Chunks of 48 with G*M = 32 rows (wave pairs) and a ragged last chunk:
    417 chunks per row, folded into splits whose last one is ragged."""
    banner("multi B=4 L=20000 M=8 chunk=48")
    c = W.multi_case(4, 8, 32, 8, 20000, 128, seed=109, device=DEV)
    rows = [(0, 0, 0), (1, 7, 31), (2, 4, 16), (3, 6, 5)]
    _check(c, chunk=48, rows=rows)


@pytest.mark.parametrize("M", [4, 8])
def test_multi_row_one_million_positions_sampled(M):
    """M new tokens at the end of a cache of 2^20 + 3 positions (2,049 chunks
    of 512): one query tile and the wave pair."""
    banner(f"multi 1M M={M}")
    c = W.multi_case(1, M, 16, 4, (1 << 20) + 3, 128, seed=1208 + M, device=DEV)
    rows = [(0, 0, 0), (0, M - 1, 15), (0, M // 2, 6)]
    _check(c, chunk=512, rows=rows)


@pytest.mark.parametrize("M,L,chunk", [(4, 100, 128), (8, 100, 128), (4, 1000, 128),
                                       (8, 1000, 128), (8, 300, 32)])
def test_multi_row_more_rows_than_wave_slots(M, L, chunk):
    """More (sequence, kv-head) rows than the device runs at once (8,192 or
    2,048 rows of G = 4 heads; 1,024 wave slots for one query tile, 1,024
    wave pairs for two): every wave or pair takes several units in a row,
    holds finished partials, crosses from one row to the next and prefetches
    the next unit's query and keys; with 300 positions in chunks of 32 a
    split of 5 chunks crosses rows mid-way.  Sampled rows, first and last
    sequences included."""
    banner(f"multi many rows M={M} L={L} chunk={chunk}")
    B = 256 if L <= 128 else (64 if L == 1000 else 48)
    c = W.multi_case(B, M, 128, 32, L, 128, seed=1300 + M + L, device=DEV)
    rows = [(0, 0, 0), (0, M - 1, 127), (B // 2, M // 2, 64), (B // 2 + 1, 1, 3),
            (B - 1, M - 1, 127), (B - 1, 0, 77)]
    _check(c, chunk=chunk, rows=rows)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("G,M", [(3, 1), (7, 1), (16, 1), (32, 1), (6, 1), (7, 4), (16, 2),
                                 (5, 3), (12, 2), (11, 2)])
def test_group_sizes_outside_vector_kernel(d, G, M):
    """Group sizes other than 1, 2, 4, 8 (e.g. 28 query heads over 4
    kv-heads: 7; 16 or 32 heads per kv-head) run on the matrix-core kernel,
    one token or several, one query tile (G*M <= 16) or two."""
    banner(f"multi any group d={d} G={G} M={M}")
    Hkv = 2
    c = W.multi_case(2, M, G * Hkv, Hkv, 333, d, seed=500 + G * M + d, device=DEV)
    _check(c, chunk=64)


@pytest.mark.parametrize("G", [7, 16, 32])
def test_single_query_entry_points_any_group(G):
    """fd_decode_attn, its allocation-free variant and the partials + merge
    pair take every group size up to 32 on bf16: each matches the fp64
    oracle, and the partials (one per chunk) merge to the full call's
    result."""
    banner(f"single-query entry points G={G}")
    Hkv = 2
    c = W.multi_case(3, 1, G * Hkv, Hkv, 1500, 128, seed=600 + G, device=DEV)
    q = c.q[:, 0].contiguous()
    ref, lref = omr.multi_row_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    out, lse = fd.decode_attn(q, c.k, c.v, chunk=128)
    torch.cuda.synchronize()
    assert max_err(f64(out), ref[:, 0]) <= TOLB and max_err(f64(lse), lref[:, 0]) <= TOLB
    o2, l2 = fd.decode_attn_noalloc(q, c.k, c.v, chunk=128)
    torch.cuda.synchronize()
    assert max_err(f64(o2), ref[:, 0]) <= TOLB and max_err(f64(l2), lref[:, 0]) <= TOLB
    ws, nc = fd.decode_attn_partials(q, c.k, c.v, chunk=128)
    assert nc == 12
    o_part, ml_part = fd.partial_views(ws, 3, G * Hkv, nc, 128)
    o3, l3 = fd.merge_partials(o_part, ml_part)
    torch.cuda.synchronize()
    assert max_err(f64(o3), ref[:, 0]) <= TOLB and max_err(f64(l3), lref[:, 0]) <= TOLB


def test_group_of_sixteen_full_size():
    """Sixteen query heads per kv-head at the headline cache (B 8, Hkv 8,
    L 32768; Hq 128): every row against the oracle."""
    banner("single query G=16 full size")
    c = W.multi_case(8, 1, 128, 8, 32768, 128, seed=616, device=DEV)
    out, lse = fd.decode_attn(c.q[:, 0].contiguous(), c.k, c.v, chunk=512)
    torch.cuda.synchronize()
    ref, lref = omr.multi_row_attention(f64(c.q), f64(c.k), f64(c.v), c.scale)
    assert max_err(f64(out), ref[:, 0]) <= TOLB and max_err(f64(lse), lref[:, 0]) <= TOLB
