"""Pins of the multi-row (several query tokens) oracle (CPU)."""
import numpy as np
import torch

from oracle import flash_decoding as ofd
from oracle import multi_row as omr


def _case(seed, B=2, M=3, Hq=4, Hkv=2, L=20, d=16):
    rs = np.random.default_rng(seed)
    return (rs.standard_normal((B, M, Hq, d)), rs.standard_normal((B, Hkv, L, d)),
            rs.standard_normal((B, Hkv, L, d)))


def test_matches_sdpa_with_bottom_right_causal_mask():
    q, k, v = _case(1)
    B, M, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out, lse = omr.multi_row_attention(q, k, v, 0.25)
    # library routine: SDPA in float64 with an explicit mask; token r sits at
    # position L - M + r and may see positions <= its own
    mask = torch.tensor([[j <= L - M + r for j in range(L)] for r in range(M)])
    tq = torch.tensor(q).permute(0, 2, 1, 3)                          # [B, Hq, M, d]
    tk = torch.tensor(k).repeat_interleave(G, dim=1)                  # [B, Hq, L, d]
    tv = torch.tensor(v).repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=0.25)
    assert np.abs(out - ref.permute(0, 2, 1, 3).numpy()).max() < 1e-12
    s = torch.einsum("bhmd,bhld->bhml", tq, tk) * 0.25
    s = s.masked_fill(~mask, float("-inf"))
    assert np.abs(lse - torch.logsumexp(s, -1).permute(0, 2, 1).numpy()).max() < 1e-12


def test_one_row_is_single_query_decode():
    q, k, v = _case(2, M=1)
    out, lse = omr.multi_row_attention(q, k, v, 0.3)
    o2, l2 = ofd.dense_attention(q[:, 0], k, v, 0.3)
    assert np.array_equal(out[:, 0], o2) and np.array_equal(lse[:, 0], l2)


def test_equal_scores_give_the_mean_of_the_visible_prefix():
    # q = 0: every visible score is 0, so token r returns the mean of V over
    # positions 0 .. L-M+r and lse = ln(L-M+r+1): an off-by-one in the causal
    # limit changes both
    q, k, v = _case(3, M=4, L=9)
    q[:] = 0.0
    out, lse = omr.multi_row_attention(q, k, v, 0.5)
    B, M, Hq, d = q.shape
    for r in range(M):
        n = 9 - 4 + r + 1
        for h in range(Hq):
            assert np.allclose(out[:, r, h], v[:, h // 2, :n].mean(1), atol=1e-14)
            assert np.allclose(lse[:, r, h], np.log(n), atol=1e-14)
