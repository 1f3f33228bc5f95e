"""The bench's FFD selection diagnostic (recall of the exact top-delta set and
the softmax mass the candidates keep) against a brute force in fp64 loops."""
import math

import numpy as np
import torch

import bench


def _pack(bits):
    """bool [.., L] -> int32 [.., ceil(L/32)], bit j%32 of word j/32."""
    L = bits.shape[-1]
    W = (L + 31) // 32
    words = np.zeros(bits.shape[:-1] + (W,), dtype=np.uint32)
    for j in range(L):
        words[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(j % 32)
    return torch.from_numpy(words.view(np.int32))


def _brute(q, k, scale, cand, delta):
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    rec, mass = [], []
    for b in range(B):
        for h in range(Hq):
            s = [scale * sum(float(q[b, h, i]) * float(k[b, h // G, j, i]) for i in range(d))
                 for j in range(L)]
            m = max(s)
            top = [j for j in range(L) if s[j] >= m - delta]
            rec.append(sum(1 for j in top if cand[b, h, j]) / len(top))
            w = [math.exp(x - m) for x in s]
            mass.append(sum(w[j] for j in range(L) if cand[b, h, j]) / sum(w))
    return np.array(rec), np.array(mass)


def _case(seed, B=2, Hq=4, Hkv=2, L=70, d=8):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, d, generator=g) * 2
    k = torch.randn(B, Hkv, L, d, generator=g)
    return q, k, 1 / math.sqrt(d)


def test_random_masks_match_brute_force():
    q, k, scale = _case(1)
    delta = 1.3
    rs = np.random.default_rng(2)
    cand = rs.random((2, 4, 70)) < 0.6
    cand[..., 31] = True                  # sign bit of the first word
    got = bench.selection_quality(torch, q, k, scale, _pack(cand), delta)
    rec, mass = _brute(q.double(), k.double(), scale, cand, delta)
    assert abs(got["recall_exact_topdelta_mean"] - rec.mean()) < 1e-5
    assert abs(got["recall_exact_topdelta_min"] - rec.min()) < 1e-5
    assert abs(got["softmax_mass_kept_mean"] - mass.mean()) < 1e-5
    assert abs(got["softmax_mass_kept_min"] - mass.min()) < 1e-5
    assert 0 < rec.min() < 1 and 0 < mass.min() < 1   # the case is not degenerate


def test_all_none_and_exact_sets():
    q, k, scale = _case(3)
    delta = 0.8
    L = k.shape[2]
    full = np.ones((2, 4, L), dtype=bool)
    got = bench.selection_quality(torch, q, k, scale, _pack(full), delta)
    assert got["recall_exact_topdelta_min"] == 1.0 and got["softmax_mass_kept_min"] == 1.0
    got = bench.selection_quality(torch, q, k, scale, _pack(~full), delta)
    assert got["recall_exact_topdelta_mean"] == 0.0 and got["softmax_mass_kept_mean"] == 0.0
    # C = T exactly: recall 1; the mass kept is at least that of the maximum
    s = scale * torch.einsum("bgd,bgld->bgl", q.double().view(2, 2, 2, 8).reshape(2, 4, 8),
                             k.double().repeat_interleave(2, dim=1))
    top = (s >= s.amax(-1, keepdim=True) - delta).numpy()
    got = bench.selection_quality(torch, q, k, scale, _pack(top), delta)
    assert got["recall_exact_topdelta_min"] == 1.0
    assert got["softmax_mass_kept_min"] >= 1.0 / L


def test_bit_order_pins_position():
    # one key that dominates every head: only its own bit gives recall 1
    q, k, scale = _case(4, L=40)
    k[:, :, 33] = 50.0 * q.view(2, 2, 2, 8).mean(2) / q.norm(dim=-1).view(2, 2, 2).mean(-1,
                                                                                   keepdim=True)
    one = np.zeros((2, 4, 40), dtype=bool)
    one[..., 33] = True
    got = bench.selection_quality(torch, q, k, scale, _pack(one), 0.0)
    assert got["recall_exact_topdelta_min"] == 1.0
    one[..., 33] = False
    one[..., 32] = True
    got = bench.selection_quality(torch, q, k, scale, _pack(one), 0.0)
    assert got["recall_exact_topdelta_mean"] == 0.0
