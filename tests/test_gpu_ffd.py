"""GPU parity of the FFD packer and the FFD sparse decode against the oracle.

The oracle packs keys itself; the GPU packer must produce the same bytes
(integer work: bit-exact).  The GPU FFD kernel runs on the oracle's packed
arrays (and, at full size, on its own, after their equality is checked), and
must match the oracle's output within 2e-3 plus the weight of the positions
whose 2-bit score lies within 1e-4 of the threshold, and its candidate sets
bit-exactly outside that band.
"""
import math

import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import ffd as offd
from tests.helpers import banner, f64, max_err, packed_to_device, packed_to_host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BAND = 1e-4


def _assert_pack_equal(gpu, ref, where=""):
    h = packed_to_host(gpu)
    for key in ("codes", "res"):
        assert np.array_equal(h[key], ref[key]), (key, where)
    for key in ("zs", "rs"):
        assert np.array_equal(h[key].view(np.uint16), ref[key].view(np.uint16)), (key, where)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("scale", [1.0, 0.003, 40.0])
def test_pack_bit_exact(d, scale):
    banner(f"pack d={d} scale={scale}")
    g = torch.Generator(device=DEV).manual_seed(d)
    k = (scale * torch.randn((2, 3, 257, d), generator=g, device=DEV)).to(torch.bfloat16)
    k[0, 0, 5] = 1.25                                      # constant groups
    k[0, 1, 7, :32] = torch.tensor([0.0, 3.0, 0.5, 1.5, 2.5] + [0.0] * 27)  # exact ties
    k[1, 2, 9, :] = 0.0
    gpu = fd.ffd_pack(k)
    torch.cuda.synchronize()
    ref = offd.pack_keys(f64(k).astype(np.float32))
    _assert_pack_equal(gpu, ref)


def test_pack_append_range():
    g = torch.Generator(device=DEV).manual_seed(3)
    k = torch.randn((1, 2, 300, 128), generator=g, device=DEV).to(torch.bfloat16)
    full = fd.ffd_pack(k)
    part = fd.ffd_pack(k, t_begin=0, t_end=100)
    fd.ffd_pack(k, t_begin=100, t_end=299, out=part)
    fd.ffd_pack(k, t_begin=299, t_end=300, out=part)
    torch.cuda.synchronize()
    for key in full:
        assert torch.equal(full[key], part[key]), key
    empty = fd.ffd_pack(k, t_begin=50, t_end=50)
    torch.cuda.synchronize()
    assert all(int(v.abs().sum()) == 0 for v in empty.values())


def _row_check(q, packed_host, v64, b, h, G, scale, delta, n_sink, n_local, out, lse, cand,
               pmax):
    sub = {key: arr[b, h // G] for key, arr in packed_host.items()}
    K2, Kh = offd.dequant(sub, q.shape[-1])
    r = offd.ffd_row(q[b, h], K2, Kh, v64[b, h // G], scale, delta, n_sink, n_local)
    L = K2.shape[0]
    near = np.abs(r["scan"] - (r["mhat"] - delta)) <= BAND
    if cand is not None:
        got = np.unpackbits(cand[b, h].view(np.uint8), bitorder="little")[:L].astype(bool)
        bad = (got != r["cand"]) & ~near
        assert not bad.any(), (b, h, np.nonzero(bad)[0][:10])
    # output: 2e-3 plus the largest effect the near-threshold positions can have
    sel = r["cand"]
    M = r["refined"][sel].max()
    den = np.exp(r["refined"][sel] - M).sum()
    vmax = np.abs(v64[b, h // G]).max(1)
    extra = float((np.exp(r["refined"][near] - M) / den * 2 * (vmax[near] + 4.0)).sum())
    assert max_err(out[b, h], r["out"]) <= 2e-3 + extra
    assert abs(lse[b, h] - r["lse"]) <= 2e-3 + extra
    if pmax is not None:
        assert abs(pmax[b, h] - r["mhat"]) <= 1e-4
    return r


@pytest.mark.parametrize("d,G", [(128, 4), (64, 1), (128, 8), (64, 2)])
@pytest.mark.parametrize("delta", [0.5, 5.0, 7.0])
def test_ffd_matches_oracle(d, G, delta):
    banner(f"ffd d={d} G={G} delta={delta}")
    Hq = 16 if G == 8 else 8
    c = W.ffd_case(2, Hq, Hq // G, 3000, d, n_sink=4, n_local=64, chunk=512, seed=d + G,
                   device=DEV)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    pk = packed_to_device(ph, DEV)
    out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, pk, c.v, delta, c.n_sink, c.n_local,
                                                chunk=c.chunk, want_mask=True,
                                                want_pseudo_max=True)
    torch.cuda.synchronize()
    q, v64 = f64(c.q), f64(c.v)
    o, l_, cm, pm = f64(out), f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax)
    for b in range(2):
        for h in range(Hq):
            _row_check(q, ph, v64, b, h, G, c.scale, delta, c.n_sink, c.n_local, o, l_, cm, pm)


@pytest.mark.parametrize("L,n_sink,n_local,chunk", [
    (1, 4, 64, 32), (40, 4, 64, 32), (100, 0, 16, 64), (100, 8, 0, 32), (1000, 4, 64, 1024),
    (1025, 1, 1, 1024), (513, 4, 64, 256)])
def test_ffd_lengths_and_anchors(L, n_sink, n_local, chunk):
    banner(f"ffd L={L} sinks={n_sink} local={n_local} chunk={chunk}")
    c = W.ffd_case(1, 8, 2, L, 128, n_sink=n_sink, n_local=n_local, chunk=chunk, seed=L,
                   device=DEV)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, packed_to_device(ph, DEV), c.v, 3.0,
                                                n_sink, n_local, chunk=chunk, want_mask=True,
                                                want_pseudo_max=True)
    torch.cuda.synchronize()
    q, v64 = f64(c.q), f64(c.v)
    for h in range(8):
        _row_check(q, ph, v64, 0, h, 4, c.scale, 3.0, n_sink, n_local, f64(out), f64(lse),
                   cand.cpu().numpy().view(np.uint32), f64(pmax))


def test_ffd_infinite_delta_is_dense_over_refined_keys():
    c = W.ffd_case(1, 8, 2, 2000, 128, chunk=256, seed=31, device=DEV)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    out, lse, cand, _ = fd.ffd_sparse_decode(c.q, packed_to_device(ph, DEV), c.v, math.inf,
                                             chunk=256, want_mask=True)
    torch.cuda.synchronize()
    assert int(cand.cpu().numpy().view(np.uint32)[:, :, :62].astype(np.uint64).sum()) == \
        8 * 62 * 0xFFFFFFFF
    _, Kh = offd.dequant(ph, 128)
    from oracle import flash_decoding as ofd
    ref, lref = ofd.dense_attention(f64(c.q), Kh, f64(c.v), c.scale)
    assert max_err(f64(out), ref) <= 2e-3 and max_err(f64(lse), lref) <= 2e-3


def test_ffd_only_anchor_survives():
    # threshold above every 2-bit score (delta = 0 on keys where only the
    # residual carries the signal): the set is {j*} and out = V[j*].
    L, d = 64, 128
    q = torch.zeros((1, 1, d), dtype=torch.bfloat16, device=DEV)
    q[0, 0, 0] = 1.0
    k = torch.zeros((1, 1, L, d), dtype=torch.bfloat16, device=DEV)
    k[..., 1] = 8.0
    k[0, 0, 2, 0] = 1.0
    g = torch.Generator(device=DEV).manual_seed(5)
    v = torch.randn((1, 1, L, d), generator=g, device=DEV).to(torch.bfloat16)
    ph = offd.pack_keys(f64(k).astype(np.float32))
    out, lse, cand, pmax = fd.ffd_sparse_decode(q, packed_to_device(ph, DEV), v, 0.0, 4, 4,
                                                chunk=32, want_mask=True, want_pseudo_max=True)
    torch.cuda.synchronize()
    assert cand.cpu().numpy().view(np.uint32)[0, 0].tolist() == [1 << 2, 0]
    assert max_err(f64(out[0, 0]), f64(v[0, 0, 2])) <= 1e-6


def test_ffd_config5_full_size_sampled():
    banner("ffd config5 full size")
    c = W.config_case(5, device=DEV)
    gpu_pack = fd.ffd_pack(c.k)
    torch.cuda.synchronize()
    G = 4
    picks = [(0, 0), (1, 5), (3, 7)]
    host = packed_to_host(gpu_pack)
    q, v64 = f64(c.q), f64(c.v)
    for delta in c.deltas:
        out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, gpu_pack, c.v, delta, c.n_sink,
                                                    c.n_local, chunk=c.chunk, want_mask=True,
                                                    want_pseudo_max=True)
        torch.cuda.synchronize()
        o, l_, cm, pm = f64(out), f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax)
        for b, g in picks:
            ref = offd.pack_keys(f64(c.k[b, g]).astype(np.float32))
            sub = {key: arr[b, g] for key, arr in host.items()}
            _assert_pack_equal({key: val[b, g] for key, val in gpu_pack.items()}, ref,
                               where=(b, g))
            for h in (g * G, g * G + 3):
                packed_ref = {key: np.broadcast_to(ref[key], (4, 8) + ref[key].shape)
                              for key in ref}
                _row_check(q, packed_ref, v64, b, h, G, c.scale, delta, c.n_sink, c.n_local,
                           o, l_, cm, pm)
        assert torch.isfinite(out).all()


def test_ffd_peaked_workload_sampled():
    # Sharp, group-correlated queries: most positions are dropped, so the
    # compaction and the per-head masks really matter.
    banner("ffd peaked workload")
    c = W.config_case(6, device=DEV, L=16384)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    pk = packed_to_device(ph, DEV)
    G = 4
    q, v64 = f64(c.q), f64(c.v)
    for delta in c.deltas:
        out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, pk, c.v, delta, c.n_sink, c.n_local,
                                                    chunk=c.chunk, want_mask=True,
                                                    want_pseudo_max=True)
        torch.cuda.synchronize()
        cm = cand.cpu().numpy().view(np.uint32)
        kept = np.unpackbits(cm.view(np.uint8), axis=-1).sum() / cm.size / 32
        assert kept < 0.4, kept
        for b, h in ((0, 0), (1, 9), (3, 30)):
            _row_check(q, ph, v64, b, h, G, c.scale, delta, c.n_sink, c.n_local, f64(out),
                       f64(lse), cm, f64(pmax))


def test_ffd_one_million_positions():
    """One sequence of 2^20 + 33 positions (1,025 chunks of 1,024, a ragged
    last one), keys packed by the oracle, every head checked in full."""
    banner("ffd 1M")
    L = (1 << 20) + 33
    c = W.ffd_case(1, 4, 1, L, 128, n_sink=4, n_local=64, chunk=1024, seed=1206, device=DEV)
    ph = offd.pack_keys(f64(c.k).astype(np.float32))
    out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, packed_to_device(ph, DEV), c.v, 5.0,
                                                c.n_sink, c.n_local, chunk=c.chunk,
                                                want_mask=True, want_pseudo_max=True)
    torch.cuda.synchronize()
    q, v64 = f64(c.q), f64(c.v)
    o, l_, cm, pm = f64(out), f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax)
    for h in range(4):
        _row_check(q, ph, v64, 0, h, 4, c.scale, 5.0, c.n_sink, c.n_local, o, l_, cm, pm)
