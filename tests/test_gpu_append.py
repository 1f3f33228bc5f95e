"""GPU parity of the cache append against the oracle (bit-exact copies), and
append -> decode on a live cache (dense, paged, FFD-packed keys)."""
import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import append as oap
from oracle import ffd as offd
from oracle import paged as opg
from tests.helpers import TOL, banner, f64, max_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _randn(shape, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(dtype)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d,M,t", [(128, 1, 0), (128, 3, 97), (64, 5, 123)])
def test_contiguous_append_bit_exact(dtype, d, M, t):
    banner(f"append contiguous d={d} M={M} t={t} {dtype}")
    B, Hkv, L_cap = 3, 2, 128
    k = _randn((B, Hkv, L_cap, d), dtype, 1)
    v = _randn((B, Hkv, L_cap, d), dtype, 2)
    kn = _randn((B, Hkv, M, d), dtype, 3)
    vn = _randn((B, Hkv, M, d), dtype, 4)
    ref_k = oap.append_contiguous(f64(k), f64(kn), t)
    ref_v = oap.append_contiguous(f64(v), f64(vn), t)
    fd.kv_append(kn, vn, k, v, t)
    torch.cuda.synchronize()
    assert np.array_equal(f64(k), ref_k) and np.array_equal(f64(v), ref_v)


def _pool(B=3, Hkv=2, page=16, d=128, max_pages=4, P=16, seed=5, dtype=torch.bfloat16):
    rs = np.random.default_rng(seed)
    table = rs.permutation(P)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    kp = _randn((P, Hkv, page, d), dtype, seed + 1)
    vp = _randn((P, Hkv, page, d), dtype, seed + 2)
    return kp, vp, table


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_paged_append_bit_exact_with_skips(dtype):
    banner(f"append paged {dtype}")
    kp, vp, table = _pool(dtype=dtype)
    table[0, 0] = -1                       # no page: positions 0..15 of seq 0 are skipped
    table[1, 2] = 99                       # not a page of the pool: skipped
    pos = np.array([3, 30, 60], dtype=np.int32)   # seq 2 runs past its 4-page row at 64
    M = 6
    kn = _randn((3, 2, M, 128), dtype, 7)
    vn = _randn((3, 2, M, 128), dtype, 8)
    ref_k = oap.append_paged(f64(kp), table, pos, f64(kn))
    ref_v = oap.append_paged(f64(vp), table, pos, f64(vn))
    fd.kv_append_paged(kn, vn, kp, vp, torch.as_tensor(table, device=DEV),
                       torch.as_tensor(pos, device=DEV))
    torch.cuda.synchronize()
    assert np.array_equal(f64(kp), ref_k) and np.array_equal(f64(vp), ref_v)


def test_paged_append_then_decode():
    """One decode step on a live paged cache: append the new token's K/V at
    position seq_len, then attend over seq_len + 1 positions."""
    banner("append paged then decode")
    kp, vp, table = _pool(seed=11)
    lens = np.array([5, 16, 47], dtype=np.int32)
    kn = _randn((3, 2, 1, 128), torch.bfloat16, 12)
    vn = _randn((3, 2, 1, 128), torch.bfloat16, 13)
    q = _randn((3, 8, 128), torch.bfloat16, 14)
    t_table = torch.as_tensor(table, device=DEV)
    fd.kv_append_paged(kn, vn, kp, vp, t_table, torch.as_tensor(lens, device=DEV))
    new_lens = torch.as_tensor(lens + 1, device=DEV)
    out, lse = fd.decode_attn_paged(q, kp, vp, t_table, new_lens, int(lens.max()) + 1, chunk=32)
    torch.cuda.synchronize()
    ref, lref = opg.paged_attention(f64(q), f64(kp), f64(vp), table, lens + 1, 16,
                                    1.0 / np.sqrt(128))
    assert max_err(f64(out), ref) <= TOL[torch.bfloat16]
    assert max_err(f64(lse), lref) <= TOL[torch.bfloat16]
    # the appended row is the one the decode saw: the gathered caches end with it
    for b in range(3):
        K = opg.gather_sequence(f64(kp), table[b], int(lens[b]) + 1, 16)
        assert np.array_equal(K[:, -1], f64(kn)[b, :, 0])


def test_contiguous_append_then_ffd_pack_range():
    """Live FFD cache: after appending M keys at position t, packing [t, t+M)
    into the existing arrays gives what packing the whole cache gives."""
    banner("append then ffd pack")
    c = W.ffd_case(2, 8, 2, 512, 128, seed=15, device=DEV)
    L_cap, t, M = 512, 500, 4
    packed = fd.ffd_pack(c.k, 0, t)                     # the cache before the step
    kn = _randn((2, 2, M, 128), torch.bfloat16, 16)
    vn = _randn((2, 2, M, 128), torch.bfloat16, 17)
    fd.kv_append(kn, vn, c.k, c.v, t)
    fd.ffd_pack(c.k, t, t + M, out=packed)              # only the new rows
    whole = fd.ffd_pack(c.k, 0, t + M)
    torch.cuda.synchronize()
    for name in ("codes", "zs", "res", "rs"):
        assert torch.equal(packed[name][:, :, :t + M], whole[name][:, :, :t + M]), name
    # and the oracle packer agrees on the appended rows
    ref = offd.pack_keys(f64(kn))
    assert np.array_equal(packed["res"][:, :, t:t + M].cpu().numpy(), ref["res"])
