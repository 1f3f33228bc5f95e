"""GPU parity of the paged and fixed-maximum paths against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import flash_decoding as ofd
from oracle import paged as opg
from oracle import unified as oun
from tests.helpers import TOL, banner, f32, f64, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _paged_run(c, max_len=None):
    max_len = int(max(c.meta["lens"])) if max_len is None else max_len
    out, lse = fd.decode_attn_paged(c.q, c.k_pool, c.v_pool, c.block_table, c.seq_lens,
                                    max_len, chunk=c.chunk)
    torch.cuda.synchronize()
    return out, lse


def _paged_ref(c, rows=None):
    # the pools as exact fp32 copies (bf16 and fp32 values are fp32): half
    # the host memory of fp64, and the oracle's gather widens each
    # sequence's rows to fp64
    return opg.paged_attention(f64(c.q), f32(c.k_pool), f32(c.v_pool),
                               c.block_table.cpu().numpy(), c.seq_lens.cpu().numpy(), c.page,
                               c.scale, rows=rows)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d,G", [(128, 4), (64, 1), (128, 8), (64, 2)])
def test_paged_ragged(dtype, d, G):
    banner(f"paged d={d} G={G} {dtype}")
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000]
    Hq = 16 if G == 8 else 8
    c = W.paged_case(len(lens), Hq, Hq // G, d, 0, 1024, page=16, chunk=64, seed=d + G,
                     device=DEV, lens=lens)
    if dtype == torch.float32:
        c.q, c.k_pool, c.v_pool = c.q.float(), c.k_pool.float(), c.v_pool.float()
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= TOL[dtype]
    assert max_err(f64(lse), lref) <= TOL[dtype]
    assert torch.all(out[0] == 0) and torch.all(torch.isinf(lse[0]))


@pytest.mark.parametrize("page,chunk", [(8, 64), (32, 128), (64, 64), (8, 1024), (16, 2048)])
def test_paged_page_sizes(page, chunk):
    c = W.paged_case(4, 8, 2, 128, 100, 700, page=page, chunk=chunk, seed=page, device=DEV)
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3


def test_paged_equals_dense_and_relabel_invariant():
    lens = [300, 300, 300]
    c = W.paged_case(3, 8, 2, 128, 0, 512, page=16, chunk=128, seed=9, device=DEV, lens=lens)
    out, lse = _paged_run(c)
    # contiguous copy of the same sequences
    pg = c.block_table[:, :19].long()                    # 19 pages of 16 cover 300
    k = c.k_pool[pg].permute(0, 2, 1, 3, 4).reshape(3, 2, 19 * 16, 128)[:, :, :300].contiguous()
    v = c.v_pool[pg].permute(0, 2, 1, 3, 4).reshape(3, 2, 19 * 16, 128)[:, :, :300].contiguous()
    o2, l2 = fd.decode_attn(c.q, k, v, chunk=128)
    # same values, same chunks, same batch depth and summation order: bitwise
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    # relabelling the pool's pages: same arithmetic, bitwise equal
    P = c.k_pool.shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(1)).to(DEV)
    inv = torch.argsort(perm)
    table = torch.where(c.block_table >= 0, inv[c.block_table.clamp(min=0).long()].int(),
                        c.block_table)
    o3, l3 = fd.decode_attn_paged(c.q, c.k_pool[perm].contiguous(), c.v_pool[perm].contiguous(),
                                  table.contiguous(), c.seq_lens, 300, chunk=128)
    assert torch.equal(out, o3) and torch.equal(lse, l3)


@pytest.mark.parametrize("B", [129, 300])
def test_paged_many_sequences(B):
    """More sequences than the partial chunks are sorted for (they are then
    taken in sequence order): empty ones, exact chunk multiples, ragged."""
    banner(f"paged many sequences B={B}")
    rs = np.random.default_rng(B)
    lens = rs.integers(0, 400, size=B)
    lens[::7] = 0
    lens[3::11] = 64 * rs.integers(1, 6, size=len(lens[3::11]))
    c = W.paged_case(B, 8, 2, 128, 0, 400, page=16, chunk=64, seed=B, device=DEV,
                     lens=lens)
    out, lse = _paged_run(c, max_len=400)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3


def test_paged_equal_remainders():
    """Sequences whose last chunks are equally long (ties in the
    longest-first order of the partial chunks)."""
    banner("paged equal remainders")
    lens = [128 * k + 17 for k in range(1, 9)] + [128 * k + 90 for k in range(1, 9)] + [256, 0]
    c = W.paged_case(len(lens), 8, 2, 128, 0, 2000, page=16, chunk=128, seed=5, device=DEV,
                     lens=lens)
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3


def test_paged_config3_full_size():
    """Paged ragged workload (16 sequences, lengths U[1024, 131072], page 16,
    chunk 1024): every one of the 512 (sequence, head) rows."""
    banner("paged config3 full size")
    c = W.config_case(3, device=DEV)
    out, lse = _paged_run(c)
    assert torch.isfinite(out).all()
    ref, lref = _paged_ref(c)
    eo, el = max_err(f64(out), ref), max_err(f64(lse), lref)
    assert eo <= 2e-3 and el <= 2e-3, (eo, el)


def _unified_check(c, phi, margin_hi, margin_lo):
    out, lse, flags = fd.decode_attn_unified_max(c.q, c.k, c.v, phi, chunk=c.chunk,
                                                 margin_hi=margin_hi, margin_lo=margin_lo)
    torch.cuda.synchronize()
    q, k, v = f64(c.q), f64(c.k), f64(c.v)
    ref, lref, rflags = oun.unified_attention(q, k, v, c.scale, phi, margin_hi, margin_lo,
                                              c.chunk)
    tol = TOL[c.q.dtype]
    assert max_err(f64(out), ref) <= tol and max_err(f64(lse), lref) <= tol
    # flags agree except where a chunk maximum sits within 1e-4 of a bound
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    got = flags.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            s = c.scale * (k[b, h // G] @ q[b, h])
            for ci, (a0, a1) in enumerate(ofd.chunk_bounds(k.shape[2], c.chunk)):
                mx = s[a0:a1].max()
                near = min(abs(mx - (phi + margin_hi)), abs(mx - (phi - margin_lo))) <= 1e-4
                if not near:
                    assert got[b, h, ci] == rflags[b, h, ci], (b, h, ci)
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("phi", [3.0, 0.0, 60.0, -60.0])
def test_unified_any_phi_is_exact(dtype, phi):
    banner(f"unified phi={phi} {dtype}")
    c = W.dense_case(2, 8, 2, 1500, 128, dtype, 256, seed=21, device=DEV)
    flags = _unified_check(c, phi, 10.0, 40.0)
    if phi >= 60.0 or phi <= -60.0:
        assert flags.all()          # every chunk out of range -> all recomputed
    if phi == 3.0:
        assert not flags.any()


def test_unified_tight_margins_mixed_flags():
    c = W.dense_case(1, 8, 8, 4000, 64, "f32", 128, seed=22, device=DEV)
    flags = _unified_check(c, 1.0, 1.5, 1.0)
    assert flags.any() and not flags.all()


def test_unified_overflow_plant():
    # one key 100 above phi: exp(100) overflows fp32 without the fallback
    c = W.dense_case(1, 4, 1, 2048, 64, "f32", 256, seed=23, device=DEV)
    phi = 2.0
    qh = f64(c.q)[0, 0]
    key = (phi + 100.0) / c.scale * qh / (qh @ qh)
    c.k[0, 0, 1234] = torch.as_tensor(key, dtype=torch.float32, device=DEV)
    flags = _unified_check(c, phi, 10.0, 40.0)
    assert flags[0, 0, 1234 // 256] == 1


def test_unified_many_units_per_wave():
    """Chunks of 16 over L 32768: 16 units per wave, so held partials and
    their range flags are written mid-run; tight margins mix flagged and
    unflagged chunks."""
    banner("unified many units per wave")
    c = W.dense_case(2, 16, 4, 32768, 128, "bf16", 16, seed=29, device=DEV)
    flags = _unified_check(c, 1.0, 1.0, 1.5)
    assert 0 < int(flags.sum()) < flags.size


def test_unified_config4_full_size():
    """Fixed-maximum workload (B 4, L 65536, chunk 512, 2 heads planted
    above phi): every (sequence, head) row against the dense definition,
    every chunk flag against the oracle's outside the 1e-4 band, and only the
    planted chunks flagged."""
    banner("unified config4 full size")
    c = W.config_case(4, device=DEV)
    flags = _unified_check(c, c.phi, c.margin_hi, c.margin_lo)
    planted = {(b, h, j // c.chunk) for b, h, j in c.overflow_heads}
    got = {tuple(x) for x in np.argwhere(flags).tolist()}
    assert got == planted


@pytest.mark.parametrize("d", [64, 128])
def test_paged_merge_of_many_chunks(d):
    """Paged rows of 0 to 257 chunks of 16 positions: the merge for rows of
    many chunks reads each row's own chunk count from the sequence lengths."""
    banner(f"paged many chunks d={d}")
    lens = [0, 1, 16, 17, 2047, 2048, 16 * 256 + 5, 300]
    c = W.paged_case(len(lens), 8, 2, d, 0, max(lens), page=16, chunk=16, seed=7 + d,
                     device=DEV, lens=lens)
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    keep = np.asarray(lens) > 0
    assert torch.all(out[~torch.as_tensor(keep, device=out.device)] == 0)
    eo = max_err(f64(out)[keep], ref[keep])
    el = max_err(f64(lse)[keep], lref[keep])
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


def test_paged_one_million_positions():
    """A pool holding one sequence of 2^20 + 5 positions (65,537 pages of 16)
    beside a short one: 1,025 chunks of 1,024 for the long row, 3 for the
    short one, in one call.  Every row checked."""
    banner("paged 1M")
    lens = [(1 << 20) + 5, 3000]
    c = W.paged_case(2, 8, 2, 128, 0, max(lens), page=16, chunk=1024, seed=1205, device=DEV,
                     lens=lens)
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3
    assert torch.isfinite(out).all()


def test_unified_one_million_positions():
    """Fixed maximum over one sequence of 2^20 + 9 positions (2,049 chunks of
    512); tight margins mix chunks inside and outside the range."""
    banner("unified 1M")
    c = W.dense_case(1, 8, 2, (1 << 20) + 9, 128, "bf16", 512, seed=1207, device=DEV)
    flags = _unified_check(c, 1.0, 1.0, 1.5)
    assert 0 < int(flags.sum()) < flags.size


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("page", [16, 64])
def test_paged_group_of_eight_long_calls(dtype, page):
    """G = 8 over a ragged paged cache with 1,024 or more (sequence, kv-head,
    chunk) units: bf16 takes the matrix-core kernel (pages divided over the
    workers), fp32 the vector kernel; every row against the oracle."""
    banner(f"paged G=8 long call {dtype} page={page}")
    c = W.paged_case(16, 64, 8, 128, 1024, 16384, page=page, chunk=512, seed=1400 + page,
                     device=DEV)
    if dtype == torch.float32:
        c.q, c.k_pool, c.v_pool = c.q.float(), c.k_pool.float(), c.v_pool.float()
    out, lse = _paged_run(c)
    ref, lref = _paged_ref(c)
    assert max_err(f64(out), ref) <= TOL[dtype]
    assert max_err(f64(lse), lref) <= TOL[dtype]


@pytest.mark.parametrize("phi,margin_hi,margin_lo", [(3.0, 0.5, 0.5), (0.0, 10.0, 40.0)])
def test_unified_group_of_eight_long_call(phi, margin_hi, margin_lo):
    """bf16 with G = 8 on a call of 1,024 units computes every chunk with its
    own maximum on the matrix-core kernel and derives the range flags from
    the chunk maxima: the dense result and the oracle's flags (narrow
    margins flag many chunks on both sides)."""
    banner(f"unified G=8 long call phi={phi}")
    c = W.dense_case(8, 64, 8, 8192 - 5, 128, "bf16", 512, seed=1500, device=DEV)
    flags = _unified_check(c, phi, margin_hi, margin_lo)
    if margin_hi < 1:
        assert 0 < flags.mean() < 1
