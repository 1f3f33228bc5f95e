"""GPU parity of multi-row decode over a paged cache (several new tokens per
sequence, any group size up to 32 query rows per kv-head, block table and
device lengths) against the fp64 oracle, every row."""
import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import paged as opg
from tests.helpers import TOL, banner, f64, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOLB = TOL[torch.bfloat16]


def _host_pools(c):
    return c.k_pool.float().cpu().numpy(), c.v_pool.float().cpu().numpy()


def _check(c, max_seq_len, chunk, rows=None):
    out, lse = fd.decode_attn_multi_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                          max_seq_len, chunk=chunk)
    torch.cuda.synchronize()
    kp, vp = _host_pools(c)
    ref, lref = opg.paged_multi_row_attention(f64(c.q), kp, vp, c.block_table.cpu().numpy(),
                                              c.seq_lens.cpu().numpy(), c.page, c.scale,
                                              rows=rows)
    if rows is None:
        assert max_err(f64(out), ref) <= TOLB
        assert max_err(f64(lse), lref) <= TOLB
    else:
        for b, r, h in rows:
            assert max_err(f64(out[b, r, h]), ref[b, r, h]) <= TOLB, (b, r, h)
            assert abs(float(lse[b, r, h]) - lref[b, r, h]) <= TOLB, (b, r, h)
    return out, lse


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("G,M", [(4, 4), (4, 8), (7, 4), (16, 1), (16, 2), (8, 2), (2, 3),
                                 (32, 1), (4, 1)])
@pytest.mark.parametrize("page", [16, 64])
def test_paged_multi_row(d, G, M, page):
    """Ragged lengths: empty, shorter than the token count, a page or chunk
    edge either side, several chunks (one query tile for G*M <= 16, the wave
    pair above; M = 1 with G = 4 takes the paged single-query kernel)."""
    banner(f"paged multi d={d} G={G} M={M} page={page}")
    Hkv = 2
    lens = [0, 3, M, 127, 128, 129, 700]
    c = W.paged_case(len(lens), G * Hkv, Hkv, d, 0, 700, page=page, chunk=128,
                     seed=40 + G * M + page + d, device=DEV, lens=lens, M=M)
    out, lse = _check(c, max(lens), 128)
    assert torch.all(out[0] == 0) and torch.all(torch.isinf(lse[0]))


@pytest.mark.parametrize("chunk", [16, 64, 1024])
def test_paged_multi_row_chunks(chunk):
    """Splits of one page (chunk 16), of several, and longer than most
    sequences (the chunk is the split on a paged cache)."""
    banner(f"paged multi chunk={chunk}")
    lens = [1, 17, 300, 1000, 2500]
    c = W.paged_case(len(lens), 16, 2, 128, 0, 2500, page=16, chunk=chunk, seed=70 + chunk,
                     device=DEV, lens=lens, M=4)
    _check(c, max(lens), chunk)


def test_paged_multi_row_equals_contiguous_on_identity_table():
    """Pages in order (block table b*n + i) hold the contiguous cache: the
    paged kernels then do the contiguous kernels' arithmetic, bit for bit
    (192 units, fewer than the device runs at once, so the contiguous call
    keeps the caller's chunk as its split too)."""
    banner("paged multi identity table")
    B, M, Hq, Hkv, L, d, page = 3, 8, 32, 8, 4096, 128, 16
    c = W.multi_case(B, M, Hq, Hkv, L, d, chunk=512, seed=77, device=DEV)
    npg = L // page
    pool_k = c.k.view(B, Hkv, npg, page, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, page, d)
    pool_v = c.v.view(B, Hkv, npg, page, d).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, page, d)
    table = torch.arange(B * npg, dtype=torch.int32, device=DEV).view(B, npg)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    o1, l1 = fd.decode_attn_multi(c.q, c.k, c.v, chunk=512)
    o2, l2 = fd.decode_attn_multi_paged(c.q, pool_k.contiguous(), pool_v.contiguous(), table,
                                        lens, L, chunk=512)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_multi_row_one_token_is_paged_decode():
    c = W.paged_case(4, 8, 2, 128, 0, 900, page=32, chunk=256, seed=81, device=DEV,
                     lens=[0, 5, 256, 900], M=1)
    o1, l1 = fd.decode_attn_multi_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                        900, chunk=256)
    o2, l2 = fd.decode_attn_paged(c.q[:, 0].contiguous(), c.k_pool, c.v_pool, c.block_table,
                                  c.seq_lens, 900, chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, 0], o2) and torch.equal(l1[:, 0], l2)


def test_paged_multi_row_empty_cache():
    c = W.paged_case(2, 8, 2, 128, 0, 0, page=16, chunk=64, seed=82, device=DEV, lens=[0, 0],
                     M=4)
    out, lse = fd.decode_attn_multi_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                          0, chunk=64)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isinf(lse)) and torch.all(lse < 0)


def test_paged_multi_row_repeatable():
    c = W.paged_case(6, 32, 8, 128, 1, 3000, page=16, chunk=256, seed=83, device=DEV, M=8)
    outs = [fd.decode_attn_multi_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                       3000, chunk=256) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


@pytest.mark.parametrize("M", [4, 8])
def test_paged_multi_row_long_ragged_sampled(M):
    """Sixteen sequences of U[1024, 131072] positions in pages of 16 (the
    paged workload's recipe) with M new tokens each: every token and head of
    the shortest and the longest sequence against the oracle."""
    banner(f"paged multi long ragged M={M}")
    c = W.paged_case(16, 32, 8, 128, 1024, 131072, page=16, chunk=512, seed=103, device=DEV,
                     M=M)
    lens = c.seq_lens.cpu().numpy()
    picks = [int(np.argmin(lens)), int(np.argmax(lens))]
    rows = [(b, r, h) for b in picks for r in range(M) for h in range(32)]
    _check(c, int(lens.max()), 512, rows=rows)


@pytest.mark.parametrize("M", [4, 8])
def test_paged_multi_row_one_million_positions(M):
    """A sequence of 2^20 + 77 positions (65,541 pages of 16) beside a short
    one, M new tokens, chunk 1024: 1,025 chunks per row, so the merge walks
    its tiles of 256 chunks; the one-tile kernel (M = 4) and the wave pair
    (M = 8) each divide the 131,120 pages of both kv-heads over their
    workers.  Every token and head against the oracle."""
    banner(f"paged multi 1M M={M}")
    lens = [(1 << 20) + 77, 300]
    c = W.paged_case(2, 8, 2, 128, 0, lens[0], page=16, chunk=1024, seed=104 + M, device=DEV,
                     lens=lens, M=M)
    _check(c, lens[0], 1024)


def test_paged_multi_row_many_short_units():
    """Forty-eight sequences of 1-600 positions, M = 8 (32 rows per kv-head,
    the wave pair), chunk 64: about two units and a cut split per worker, so
    each worker writes one unit's partials beside the next unit's loads
    several times and the fix-up folds the cut parts.  Every row against
    the oracle."""
    banner("paged multi many short units M=8")
    rs = np.random.RandomState(105)
    lens = [int(x) for x in rs.randint(1, 601, size=48)]
    c = W.paged_case(len(lens), 32, 8, 128, 0, max(lens), page=16, chunk=64, seed=105,
                     device=DEV, lens=lens, M=8)
    _check(c, max(lens), 64)
