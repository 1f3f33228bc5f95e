"""The seeded input generators (CPU only, reduced sizes)."""
import math

import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_round_to_nearest_even():
    # the generators store bf16 through torch's conversion; it must be RNE
    x = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20,
                      float("inf"), float("-inf")])
    y = x.to(torch.bfloat16).float().tolist()
    assert y[:4] == [1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7]
    assert y[4] == float("inf") and y[5] == float("-inf")
    assert math.isnan(torch.tensor([float("nan")]).to(torch.bfloat16).float().item())


def test_dense_case_shapes_and_determinism():
    a = W.dense_case(2, 8, 2, 100, 64, "bf16", 32, seed=7)
    b = W.dense_case(2, 8, 2, 100, 64, "bf16", 32, seed=7)
    c = W.dense_case(2, 8, 2, 100, 64, "bf16", 32, seed=8)
    assert a.q.shape == (2, 8, 64) and a.k.shape == (2, 2, 100, 64)
    assert a.k.dtype == torch.bfloat16 and a.scale == 0.125
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.q, b.q)
    assert not torch.equal(a.k, c.k)
    f = W.dense_case(1, 4, 4, 10, 64, "f32", seed=1)
    assert f.k.dtype == torch.float32


def test_config_table():
    assert W.CONFIGS[2]["L"] == 32768 and W.CONFIGS[2]["chunk"] == 512
    assert W.CONFIGS[1]["dtype"] == "f32"
    small = W.config_case(2, L=256, B=1)
    assert small.k.shape == (1, 8, 256, 128)


def test_paged_case_structure():
    c = W.paged_case(3, 8, 2, 32, 20, 70, page=16, chunk=32, seed=3)
    lens = c.seq_lens.tolist()
    assert all(20 <= L <= 70 for L in lens)
    n = [(L + 15) // 16 for L in lens]
    used = np.concatenate([c.block_table[b, :n[b]].numpy() for b in range(3)])
    assert sorted(used.tolist()) == list(range(sum(n)))         # a permutation
    for b in range(3):
        assert np.all(c.block_table[b, n[b]:].numpy() == -1)
        last = c.block_table[b, n[b] - 1].item()
        tail = lens[b] - (n[b] - 1) * 16
        assert torch.all(c.k_pool[last, :, tail:] == 0)
        assert torch.all(c.k_pool[last, :, :tail] != 0)
    c2 = W.paged_case(3, 8, 2, 32, 20, 70, page=16, chunk=32, seed=3)
    assert torch.equal(c.k_pool, c2.k_pool) and torch.equal(c.block_table, c2.block_table)


def test_paged_case_explicit_lengths_with_empty():
    c = W.paged_case(2, 4, 1, 16, 0, 40, page=16, seed=1, lens=[0, 33])
    assert c.seq_lens.tolist() == [0, 33]
    assert np.all(c.block_table[0].numpy() == -1)


def test_unified_case_overflow_plant():
    c = W.unified_case(2, 8, 2, 2048, 64, chunk=256, over_frac=0.1, seed=4)
    assert len(c.over if hasattr(c, "over") else c.overflow_heads) == 2
    G = 4
    for b, h, j in c.overflow_heads:
        s = float(c.k[b, h // G, j].double() @ c.q[b, h].double()) * c.scale
        assert s == pytest.approx(c.phi + 15.0, abs=0.2)
        assert s > c.phi + c.margin_hi
    # phi sits at the top of the ordinary score range
    s_all = torch.matmul(c.k.double(), c.q.double().view(2, 2, 4, 64).transpose(-1, -2)) * c.scale
    assert 3.0 < c.phi < 15.0
    assert float(s_all.max()) > c.phi + 10


def test_unified_case_plants_raise_scores():
    c = W.unified_case(1, 4, 1, 4096, 64, chunk=512, over_frac=0.0, seed=5, phi=1.0)
    s = (c.k[0, 0].double() @ c.q[0].double().T) * c.scale      # [L, Hq]
    top = s.max(0).values
    # planted positions are raised by 0.5*|q|^2*scale (about 2.8 at d = 64)
    shift = 0.5 * (c.q[0].double() ** 2).sum(1) * c.scale
    assert torch.all(top > shift)


def test_ffd_case_sinks_and_needles():
    c = W.ffd_case(2, 8, 2, 4096, 64, seed=6)
    s = torch.einsum("bgld,bghd->bghl", c.k.double(),
                     c.q.double().view(2, 2, 4, 64)) * c.scale
    sink_mean = s[..., :4].mean().item()
    assert 2.0 < sink_mean < 4.0
    rest = s[..., 4:-64]
    frac_high = (rest > 3.5).double().mean().item()
    assert 0.005 < frac_high < 0.03


def test_ffd_peaked_queries_share_group_direction():
    c = W.ffd_case(1, 8, 2, 256, 64, seed=3, q_scale=5.0, q_shared=0.95)
    q = c.q.float()
    assert 4.0 < float(q.std()) < 6.0
    cos = torch.nn.functional.cosine_similarity(q[0, 0], q[0, 1], dim=0)
    assert float(cos) > 0.8                       # same group: nearly aligned
    cos2 = torch.nn.functional.cosine_similarity(q[0, 0], q[0, 4], dim=0)
    assert abs(float(cos2)) < 0.5                 # other group: unrelated
    base = W.config_case(5, L=256, B=1)
    assert base.q.float().std() < 1.5
