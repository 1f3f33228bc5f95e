"""GPU parity of the FFD packer and the FFD sparse decode against the oracle.

The oracle packs keys itself; the GPU packer must produce the same bytes
(integer work: bit-exact).  The GPU FFD kernel runs on the oracle's packed
arrays (and, at full size, on its own, after their equality is checked), and
must match the oracle's output within 2e-3 plus the largest change that moving
the positions whose 2-bit score lies within 1e-4 of the threshold into or out
of the set can cause (an exact bound from oracle values, `toggle_bound`), and
its candidate sets bit-exactly outside that band.
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


def toggle_bound(r, near, V):
    """Largest change of out (max norm) and of lse that moving the positions
    in ``near`` into or out of the oracle's candidate set can cause.

    With the oracle's set C, M = max_C s^, Z = sum_C e^(s^ - M), O its output
    and w_j = e^(s^_j - M) / Z, a set that drops D (within C) and adds A
    (outside it) has output O' with
        O' - O = (sum_A w_j (V_j - O) - sum_D w_j (V_j - O)) / (1 - w(D) + w(A))
    and lse' - lse = ln(1 - w(D) + w(A)), so over every such D and A of the
    near positions N (j* is always kept, so it is never dropped):
        |O' - O| <= sum_N w_j |V_j - O|_inf / (1 - w(N & C)),
        |lse' - lse| <= max(-ln(1 - w(N & C)), ln(1 + w(N - C))).
    Every quantity is the oracle's (r) or an input (V); nothing comes from
    the GPU."""
    idx = np.nonzero(near)[0]
    idx = idx[idx != r["jstar"]]
    if idx.size == 0:
        return 0.0, 0.0
    sel = r["cand"]
    M = r["refined"][sel].max()
    Z = np.exp(r["refined"][sel] - M).sum()
    w = np.exp(r["refined"][idx] - M) / Z
    inside = sel[idx]
    w_in, w_out = float(w[inside].sum()), float(w[~inside].sum())
    assert w_in < 0.5, w_in
    spread = np.abs(V[idx] - r["out"]).max(axis=1)
    d_out = float((w * spread).sum() / (1.0 - w_in))
    d_lse = float(max(-np.log1p(-w_in), np.log1p(w_out)))
    return d_out, d_lse


def _check_group(q, keys, v_group, b, g, G, scale, delta, n_sink, n_local, out, lse, cand,
                 pmax, stats=None):
    """Every query head of kv-group (b, g) against the oracle: candidate sets
    bit-exact except where the 2-bit score lies within BAND of the threshold
    (oracle values); out and lse within 2e-3 plus toggle_bound of those
    positions; the pseudo-maximum within 1e-4.  keys = the group's packed
    arrays, or their (2-bit, refined) dequantisation."""
    K2, Kh = keys if isinstance(keys, tuple) else offd.dequant(keys, q.shape[-1])
    for h in range(g * G, (g + 1) * G):
        r = offd.ffd_row(q[b, h], K2, Kh, v_group, scale, delta, n_sink, n_local)
        L = K2.shape[0]
        near = np.abs(r["scan"] - (r["mhat"] - delta)) <= BAND
        if cand is not None:
            got = np.unpackbits(cand[b, h].view(np.uint8), bitorder="little")[:L].astype(bool)
            bad = (got != r["cand"]) & ~near
            assert not bad.any(), (b, h, np.nonzero(bad)[0][:10])
        d_out, d_lse = toggle_bound(r, near, v_group)
        assert max_err(out[b, h], r["out"]) <= 2e-3 + d_out, (b, h)
        assert abs(lse[b, h] - r["lse"]) <= 2e-3 + d_lse, (b, h)
        if pmax is not None:
            assert abs(pmax[b, h] - r["mhat"]) <= 1e-4, (b, h)
        if stats is not None:
            stats["near"] = max(stats.get("near", 0), int(near.sum()))
            stats["d_out"] = max(stats.get("d_out", 0.0), d_out)
            stats["d_lse"] = max(stats.get("d_lse", 0.0), d_lse)


def _check_all(q, packed, v64, G, scale, delta, n_sink, n_local, out, lse, cand, pmax,
               stats=None):
    B, Hkv = v64.shape[0], v64.shape[1]
    for b in range(B):
        for g in range(Hkv):
            sub = {key: arr[b, g] for key, arr in packed.items()}
            _check_group(q, sub, v64[b, g], b, g, G, scale, delta, n_sink, n_local, out, lse,
                         cand, pmax, stats)


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
    _check_all(f64(c.q), ph, f64(c.v), G, c.scale, delta, c.n_sink, c.n_local, f64(out),
               f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax))


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
    _check_all(f64(c.q), ph, f64(c.v), 4, c.scale, 3.0, n_sink, n_local, f64(out), f64(lse),
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


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 1), (8, 1)])
def test_ffd_only_anchor_survives(Hq, Hkv):
    """Threshold above every 2-bit score (delta = 0 on keys where only the
    residual carries the signal): the set is {j*} and out = V[j*] bit for bit
    (its weight is exactly 1).  G = 1 runs the dot-product kernel form, G = 4
    and 8 the matrix-core form."""
    L, d = 64, 128
    q = torch.zeros((1, Hq, d), dtype=torch.bfloat16, device=DEV)
    q[0, :, 0] = 1.0
    k = torch.zeros((1, Hkv, L, d), dtype=torch.bfloat16, device=DEV)
    k[..., 1] = 8.0
    k[0, :, 2, 0] = 1.0
    g = torch.Generator(device=DEV).manual_seed(5)
    v = torch.randn((1, Hkv, L, d), generator=g, device=DEV).to(torch.bfloat16)
    ph = offd.pack_keys(f64(k).astype(np.float32))
    out, lse, cand, pmax = fd.ffd_sparse_decode(q, packed_to_device(ph, DEV), v, 0.0, 4, 4,
                                                chunk=32, want_mask=True, want_pseudo_max=True)
    torch.cuda.synchronize()
    for h in range(Hq):
        assert cand.cpu().numpy().view(np.uint32)[0, h].tolist() == [1 << 2, 0]
        assert torch.equal(out[0, h], v[0, h * Hkv // Hq, 2].float()), h


def test_ffd_config5_full_size():
    """FFD workload at full size (B 4, Hq 32, Hkv 8, d 128, L 65536, chunk
    1024), delta 5 and 7: the GPU packer's bytes equal the oracle's for the
    whole cache, and every query head matches the oracle run on them."""
    banner("ffd config5 full size")
    c = W.config_case(5, device=DEV)
    gpu_pack = fd.ffd_pack(c.k)
    torch.cuda.synchronize()
    B, Hq, d = c.q.shape
    Hkv = c.v.shape[1]
    G = Hq // Hkv
    host = packed_to_host(gpu_pack)
    for b in range(B):
        for g in range(Hkv):
            ref = offd.pack_keys(f64(c.k[b, g]).astype(np.float32))
            _assert_pack_equal({key: val[b, g] for key, val in gpu_pack.items()}, ref,
                               where=(b, g))
    q, v64 = f64(c.q), f64(c.v)
    runs = {}
    for delta in c.deltas:
        out, lse, cand, pmax = fd.ffd_sparse_decode(c.q, gpu_pack, c.v, delta, c.n_sink,
                                                    c.n_local, chunk=c.chunk, want_mask=True,
                                                    want_pseudo_max=True)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        runs[delta] = (f64(out), f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax), {})
    for b in range(B):
        for g in range(Hkv):
            keys = offd.dequant({key: arr[b, g] for key, arr in host.items()}, d)
            for delta, (o, l_, cm, pm, stats) in runs.items():
                _check_group(q, keys, v64[b, g], b, g, G, c.scale, delta, c.n_sink, c.n_local,
                             o, l_, cm, pm, stats)
    for delta, (_, _, _, _, stats) in runs.items():
        banner(f"ffd config5 delta={delta:g}: at most {stats['near']} positions of a row "
               f"within {BAND:g} of the threshold; largest allowance added to 2e-3: "
               f"out {stats['d_out']:.3e}, lse {stats['d_lse']:.3e}")


def test_ffd_peaked_workload():
    # Sharp, group-correlated queries: most positions are dropped, so the
    # compaction and the per-head masks really matter.  Every head checked.
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
        _check_all(q, ph, v64, G, c.scale, delta, c.n_sink, c.n_local, f64(out), f64(lse), cm,
                   f64(pmax))


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
    _check_all(f64(c.q), ph, f64(c.v), 4, c.scale, 5.0, c.n_sink, c.n_local, f64(out),
               f64(lse), cand.cpu().numpy().view(np.uint32), f64(pmax))
